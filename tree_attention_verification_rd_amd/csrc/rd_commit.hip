// Commit of the accepted path, the step after greedy accept: the best beam's
// verified keys and values join the KV cache and the drafter's hidden state
// is picked.  ("ReDrafter in NVIDIA TensorRT-LLM", intro: the best path is
// accepted before the next drafting round; Apple/NVIDIA ReDrafter news
// article, "RNN draft model": the drafter continues from the target's latest
// token and its last hidden state.)
#include "rd_common.h"
#include "rd_internal.h"

namespace rd {

struct CommitArgs {
    const int32_t *unpacker, *best_beam, *accept_len;
    const void *k_new, *v_new, *hidden;
    void *k_cache, *v_cache, *hidden_next;
    int32_t *kv_len;
    int W, L, P, Hkv, S;
    int row_units;  // copy units per key/value row (one KV head of one token)
    int hid_units;  // copy units per hidden row, 0 when no hidden row is picked
    // paged cache: k_cache / v_cache are pools [num_pages, Hkv, page_size, D], S = max_pages * page_size
    const int32_t *bt;  // block table [B, max_pages]
    int max_pages, page_size;
    int64_t num_pages;
};

// One workgroup per request.  Every work item of the request -- the key and
// value rows of candidates (best, 0..n) for every KV head, then the hidden
// row of candidate (best, n) -- is one copy unit in a flat index space that
// the workgroup walks with U loads in flight per thread.  The destination
// order (head, token, unit) makes the cache writes contiguous per head.
// kv_len[b] is read by every thread before the first barrier and written
// once by thread 0 after the copies, so it can be advanced in place within
// the one launch.
// With PAGED, position t goes to row t % page_size of page
// block_table[b, t / page_size].  Every page id the request would write is
// checked first: one that names no page of the pool (negative or past it)
// leaves the whole request unchanged, like an overflow, so a write never
// lands in a page the request does not own.
template <typename T, int U, bool PAGED>
__global__ __launch_bounds__(1024) void k_commit(CommitArgs a) {
    __shared__ int slot[kMaxBeamLen];
    __shared__ int pages[kMaxBeamLen];
    const int b = blockIdx.x;
    const int w = a.best_beam[b];
    const int n = a.accept_len[b];
    const int c = a.kv_len[b];
    const bool fits = w >= 0 && w < a.W && n >= 0 && n < a.L && c >= 0 && c <= a.S - (n + 1);
    const int rows = n + 1;
    int mine = 1;  // this thread's position has a page (or needs none)
    if (fits && static_cast<int>(threadIdx.x) < rows) {
        const int s = a.unpacker[(static_cast<size_t>(b) * a.W + w) * a.L + threadIdx.x];
        slot[threadIdx.x] = min(max(s, 0), a.P - 1);
        if constexpr (PAGED) {
            // c + rows <= S = max_pages * page_size, so the table index is in range
            const int t = c + static_cast<int>(threadIdx.x);
            const int32_t pg = a.bt[static_cast<size_t>(b) * a.max_pages + t / a.page_size];
            pages[threadIdx.x] = pg;
            mine = (pg >= 0 && static_cast<int64_t>(pg) < a.num_pages) ? 1 : 0;
        }
    }
    const bool ok = __syncthreads_and(mine) && fits;
    if (!ok) return;

    const int per_head = rows * a.row_units;
    const int per_tensor = a.Hkv * per_head;
    const int total = 2 * per_tensor + a.hid_units;
    const T *knew = static_cast<const T *>(a.k_new);
    const T *vnew = static_cast<const T *>(a.v_new);
    const T *hid = static_cast<const T *>(a.hidden);
    T *kc = static_cast<T *>(a.k_cache);
    T *vc = static_cast<T *>(a.v_cache);
    T *hn = static_cast<T *>(a.hidden_next);
    const size_t pbase = static_cast<size_t>(b) * a.P;

    auto locate = [&](int e, const T *&src, T *&dst) {
        if (e >= 2 * per_tensor) {  // the hidden row
            const int u = e - 2 * per_tensor;
            src = hid + (pbase + slot[n]) * a.hid_units + u;
            dst = hn + static_cast<size_t>(b) * a.hid_units + u;
            return;
        }
        const bool is_v = e >= per_tensor;
        const int e2 = is_v ? e - per_tensor : e;
        const int g = e2 / per_head;
        const int r = e2 - g * per_head;
        const int j = r / a.row_units;
        const int u = r - j * a.row_units;
        src = (is_v ? vnew : knew) + ((pbase + slot[j]) * a.Hkv + g) * a.row_units + u;
        size_t drow;
        if constexpr (PAGED) {
            const int t = c + j;
            drow = (static_cast<size_t>(pages[j]) * a.Hkv + g) * a.page_size + t % a.page_size;
        } else {
            drow = (static_cast<size_t>(b) * a.Hkv + g) * a.S + c + j;
        }
        dst = (is_v ? vc : kc) + drow * a.row_units + u;
    };

    for (int base = threadIdx.x; base < total; base += blockDim.x * U) {
        T v[U];
        T *d[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int e = base + i * static_cast<int>(blockDim.x);
            d[i] = nullptr;
            if (e < total) {
                const T *s;
                locate(e, s, d[i]);
                v[i] = *s;
            }
        }
#pragma unroll
        for (int i = 0; i < U; ++i)
            if (d[i]) *d[i] = v[i];
    }
    __syncthreads();
    if (threadIdx.x == 0) a.kv_len[b] = c + rows;
}

hipError_t launch_commit(int esize, const int32_t *unpacker, const int32_t *best_beam, const int32_t *accept_len,
                         const void *k_new, const void *v_new, const void *hidden, int B, int W, int L, int Hkv,
                         int D, int K, int S, void *k_cache, void *v_cache, int32_t *kv_len, void *hidden_next,
                         hipStream_t stream, const PagedKV *paged) {
    const bool with_hidden = hidden && hidden_next && K > 0;
    const int64_t row_bytes = static_cast<int64_t>(D) * esize;
    const int64_t hid_bytes = with_hidden ? static_cast<int64_t>(K) * esize : 0;
    uintptr_t align = reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
                      reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache);
    if (with_hidden) align |= reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(hidden_next);
    const bool wide = row_bytes % 16 == 0 && hid_bytes % 16 == 0 && align % 16 == 0;
    const int unit = wide ? 16 : 2;
    CommitArgs a{unpacker, best_beam, accept_len, k_new, v_new, with_hidden ? hidden : nullptr,
                 k_cache, v_cache, with_hidden ? hidden_next : nullptr, kv_len,
                 W, L, W * L, Hkv, S, static_cast<int>(row_bytes / unit), static_cast<int>(hid_bytes / unit),
                 nullptr, 0, 1, 1};
    if (paged) {
        a.bt = paged->block_table;
        a.max_pages = paged->max_pages;
        a.page_size = paged->page_size;
        a.num_pages = paged->num_pages;
    }
    constexpr int U = 4;
    if (wide) {
        auto kern = paged ? k_commit<u32x4, U, true> : k_commit<u32x4, U, false>;
        hipLaunchKernelGGL(kern, dim3(B), dim3(1024), 0, stream, a);
    } else {
        auto kern = paged ? k_commit<uint16_t, U, true> : k_commit<uint16_t, U, false>;
        hipLaunchKernelGGL(kern, dim3(B), dim3(1024), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace rd
