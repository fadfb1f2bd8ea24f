// Tuning knobs and the debug-mode content checks of librd.
//
// Knobs force a choice the planners otherwise make themselves (how many KV
// splits the attention uses, which tile shape the projection uses).  They
// exist so that tests can reach every code path at small sizes and so that
// measurements can compare shapes; the product default is 0 = automatic.
//
// Debug mode (rd_set_debug, or RD_DEBUG=1 in the environment when the
// library loads) makes every entry point check the device-side values it
// otherwise trusts -- lengths within their capacity, unpacker slots within
// the packed width, page ids within the pool -- before it launches its
// kernels.  The checks run as small kernels on the caller's stream, then the
// host waits for the stream and reads one flag: a call with a bad value
// returns RD_E_CONTENT and launches nothing else.  Debug mode therefore
// synchronises the host on every call and is not for production use.
#include <hip/hip_runtime.h>
#include <stdlib.h>

#include <atomic>

#include "../../include/rd.h"
#include "rd_internal.h"

namespace rd {

namespace {

std::atomic<int> g_knobs[RD_KNOB_COUNT];
std::atomic<int> g_debug{-1};  // -1: not yet read from the environment

// set to nonzero by any check that finds a value out of range
__device__ unsigned int g_content_bad;

__global__ void k_reset_flag() { g_content_bad = 0u; }

// p[i] must lie in [lo, hi) for i < n
__global__ __launch_bounds__(256) void k_check_range(const int32_t *__restrict__ p, int64_t n, int lo, int hi) {
    bool bad = false;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const int v = p[i];
        bad |= v < lo || v >= hi;
    }
    if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(&g_content_bad, 1u);
}

// block_table[b, t / page_size] must name a page of the pool for every
// cached position t < kv_len[b] (kv_len itself is checked separately, and
// clamped here so the table read stays inside row b)
__global__ __launch_bounds__(256) void k_check_table(const int32_t *__restrict__ bt, const int32_t *__restrict__ kv_len,
                                                     int max_pages, int page_size, int64_t num_pages) {
    const int b = blockIdx.x;
    const int kvl = min(max(kv_len[b], 0), max_pages * page_size);
    const int used = (kvl + page_size - 1) / page_size;
    bool bad = false;
    for (int j = threadIdx.x; j < used; j += 256) {
        const int32_t pg = bt[static_cast<size_t>(b) * max_pages + j];
        bad |= pg < 0 || static_cast<int64_t>(pg) >= num_pages;
    }
    if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(&g_content_bad, 1u);
}

}  // namespace

int knob(int which) {
    if (which < 1 || which >= RD_KNOB_COUNT) return 0;
    return g_knobs[which].load(std::memory_order_relaxed);
}

int set_knob(int which, int value) {
    if (which < 1 || which >= RD_KNOB_COUNT || value < 0) return RD_E_ARG;
    return g_knobs[which].exchange(value, std::memory_order_relaxed);
}

bool debug_checks() {
    int d = g_debug.load(std::memory_order_relaxed);
    if (d < 0) {
        const char *e = getenv("RD_DEBUG");
        const int want = (e && *e && *e != '0') ? 1 : 0;
        int expect = -1;
        g_debug.compare_exchange_strong(expect, want, std::memory_order_relaxed);
        d = g_debug.load(std::memory_order_relaxed);
    }
    return d == 1;
}

int set_debug(int on) {
    const int prev = debug_checks() ? 1 : 0;
    g_debug.store(on ? 1 : 0, std::memory_order_relaxed);
    return prev;
}

int check_contents(hipStream_t stream, const RangeCheck *checks, int n, const TableCheck *table) {
    hipLaunchKernelGGL(k_reset_flag, dim3(1), dim3(1), 0, stream);
    for (int i = 0; i < n; ++i) {
        const RangeCheck &c = checks[i];
        if (!c.p || c.n <= 0) continue;
        const int64_t blocks = (c.n + 255) / 256;
        hipLaunchKernelGGL(k_check_range, dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                           stream, c.p, c.n, c.lo, c.hi);
    }
    if (table && table->bt && table->B > 0 && table->max_pages > 0)
        hipLaunchKernelGGL(k_check_table, dim3(static_cast<unsigned>(table->B)), dim3(256), 0, stream, table->bt,
                           table->kv_len, table->max_pages, table->page_size, table->num_pages);
    if (hipGetLastError() != hipSuccess) return RD_E_HIP;
    unsigned int bad = 0;
    if (hipMemcpyFromSymbolAsync(&bad, HIP_SYMBOL(g_content_bad), sizeof(bad), 0, hipMemcpyDeviceToHost, stream) !=
            hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return RD_E_HIP;
    return bad ? RD_E_CONTENT : RD_OK;
}

}  // namespace rd

extern "C" {

int rd_set_knob(int knob, int value) { return rd::set_knob(knob, value); }

int rd_set_debug(int on) { return rd::set_debug(on); }

}  // extern "C"
