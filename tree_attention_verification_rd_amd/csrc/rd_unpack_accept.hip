// Step 3b (unpack gather) and step 4 (greedy accept) kernels.
#include <type_traits>

#include "rd_common.h"
#include "rd_internal.h"

namespace rd {

// Greedy accept: one wavefront per request, one lane per beam.  Lane w walks
// its beam while the draft at j+1 equals the target's choice at j; the best
// beam is the max of the key (match length, -w) across lanes, so ties go to
// the lowest beam.  A ragged request (bwid / blen given) uses only its first
// Wb beams and Lb positions; padding beams report match length -1, and a
// request with no beam or no position accepts nothing (-1 everywhere).
struct AcceptArgs {
    const int32_t *beams, *unpacker, *pargmax;
    int W, L;
    int32_t *match_len, *best_beam, *accept_len, *accepted;
    const int32_t *bwid, *blen;
};

__device__ __forceinline__ void accept_request(const AcceptArgs &a, int b, int lane) {
    const int W = a.W, L = a.L;
    const int P = W * L;
    const int32_t *am = a.pargmax + static_cast<size_t>(b) * P;
    auto target_at = [&](int w, int l) {
        const int slot = a.unpacker[(static_cast<size_t>(b) * W + w) * L + l];
        return am[min(max(slot, 0), P - 1)];
    };
    const int Wb = a.bwid ? min(max(a.bwid[b], 0), W) : W;
    const int Lb = a.blen ? min(max(a.blen[b], 0), L) : L;
    const bool real = lane < Wb && Lb > 0;
    int n = 0;
    if (real) {
        const int32_t *bw = a.beams + (static_cast<size_t>(b) * W + lane) * L;
        while (n < Lb - 1 && bw[n + 1] == target_at(lane, n)) ++n;
    }
    if (lane < W) a.match_len[static_cast<size_t>(b) * W + lane] = real ? n : -1;
    int key = real ? ((n << 6) | (63 - lane)) : -1;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) key = max(key, shfl_xor(key, off));
    const int best = key < 0 ? -1 : 63 - (key & 63);
    const int nbest = key < 0 ? -1 : key >> 6;
    if (lane == 0) {
        a.best_beam[b] = best;
        a.accept_len[b] = nbest;
    }
    if (lane < L) {
        int t = -1;
        if (best < 0)
            t = -1;
        else if (lane < nbest)
            t = a.beams[(static_cast<size_t>(b) * W + best) * L + lane + 1];
        else if (lane == nbest)
            t = target_at(best, nbest);
        a.accepted[static_cast<size_t>(b) * L + lane] = t;
    }
}

__global__ __launch_bounds__(64) void k_accept(AcceptArgs a) { accept_request(a, blockIdx.x, threadIdx.x); }

// Unpack, as the PyTorch `unpack` listing of the TensorRT-LLM ReDrafter blog
// ("Implementing in-Engine Validation and Drafting") defines it:
// out[b,w,l,:] = packed[b, unpacker[b,w,l], :].  A streaming row copy: each
// workgroup moves one chunk of one output row with UNROLL independent
// vector loads in flight per thread.  The B workgroups after the copy's run
// the greedy accept (the two parts are independent), saving a launch.
template <typename T, int UNROLL>
__global__ __launch_bounds__(256) void k_unpack_accept(const T *__restrict__ packed, T *__restrict__ out,
                                                       const int32_t *__restrict__ unpacker, int64_t row_elems,
                                                       int P, int WL, int nchunks, int64_t ncopy, AcceptArgs acc) {
    const int64_t blk = blockIdx.x;
    if (blk >= ncopy) {
        if (threadIdx.x < kWave) accept_request(acc, static_cast<int>(blk - ncopy), threadIdx.x);
        return;
    }
    const int64_t row = blk / nchunks;
    const int chunk = static_cast<int>(blk % nchunks);
    const int64_t b = row / WL;
    const int uslot = unpacker[row];  // -1: a padding candidate of a ragged request, unpacked as zeros
    const int slot = min(max(uslot, 0), P - 1);
    const T *s = packed + (b * P + slot) * row_elems;
    T *d = out + row * row_elems;
    const int64_t base = static_cast<int64_t>(chunk) * (256 * UNROLL) + threadIdx.x;
    T v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t i = base + u * 256;
        if (i < row_elems) v[u] = (uslot >= 0) ? s[i] : T{};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t i = base + u * 256;
        if (i < row_elems) __builtin_nontemporal_store(v[u], d + i);
    }
}

// The unpack folded into the projection (the same gather, other order).
// Each packed row is written once, by the projection, to the output row of
// its first candidate -- the lowest beam w with unpacker[b,w,l] = p, all of
// a node's candidates sharing its depth l.  k_node_rows finds those rows and
// lists, per request, the output rows still to fill afterwards: the node's
// other candidates (copied from its first) and padding candidates (zeros).
// With little prefix sharing the lists are short, and the copy kernel only
// walks them.
__global__ __launch_bounds__(256) void k_node_rows(const int32_t *__restrict__ unpacker, int W, int L,
                                                   int32_t *__restrict__ node_row, int2 *__restrict__ todo,
                                                   int32_t *__restrict__ ntodo) {
    __shared__ int first_w[kMaxBeams * kMaxBeamLen];
    __shared__ int depth[kMaxBeams * kMaxBeamLen];
    __shared__ int count;
    const int b = blockIdx.x;
    const int WL = W * L;
    const int32_t *u = unpacker + static_cast<size_t>(b) * WL;
    for (int p = threadIdx.x; p < WL; p += 256) first_w[p] = kMaxBeams;
    if (threadIdx.x == 0) count = 0;
    __syncthreads();
    for (int c = threadIdx.x; c < WL; c += 256) {
        const int p = u[c];
        if (p >= 0 && p < WL) {
            const int w = c / L;
            atomicMin(&first_w[p], w);
            depth[p] = c - w * L;  // every candidate of node p has its depth
        }
    }
    __syncthreads();
    for (int p = threadIdx.x; p < WL; p += 256)
        node_row[static_cast<size_t>(b) * WL + p] = first_w[p] < kMaxBeams ? b * WL + first_w[p] * L + depth[p] : -1;
    // output rows the projection does not write: (row, source row or -1 for zeros)
    for (int c = threadIdx.x; c < WL; c += 256) {
        const int p = u[c];
        const int src = (p >= 0 && p < WL) ? b * WL + first_w[p] * L + depth[p] : -1;
        if (src != b * WL + c) todo[static_cast<size_t>(b) * WL + atomicAdd(&count, 1)] = make_int2(b * WL + c, src);
    }
    __syncthreads();
    if (threadIdx.x == 0) ntodo[b] = count;
}

// Request b's list is cut into (entry, chunk of 256*UNROLL elements) items;
// workgroup (b, s) fills items s, s + S, ..., IB at a time, each thread with
// IB*UNROLL vector loads in flight, so a short list costs a few idle
// workgroups and a long one spreads over many without waiting on one load
// round trip per item.
template <typename T, int UNROLL, int IB>
__global__ __launch_bounds__(256) void k_unpack_dups(T *__restrict__ out, const int2 *__restrict__ todo,
                                                     const int32_t *__restrict__ ntodo, int64_t row_elems, int WL,
                                                     int nchunks, int S) {
    const int b = blockIdx.x / S;
    const int s = blockIdx.x % S;
    const int items = ntodo[b] * nchunks;
    for (int it0 = s; it0 < items; it0 += S * IB) {
        T v[IB][UNROLL];
        int2 e[IB];
        int64_t base[IB];
#pragma unroll
        for (int q = 0; q < IB; ++q) {
            const int it = it0 + q * S;
            const int j = (it < items) ? it / nchunks : 0;
            e[q] = (it < items) ? todo[static_cast<size_t>(b) * WL + j] : make_int2(-1, -1);
            base[q] = static_cast<int64_t>(it - j * nchunks) * (256 * UNROLL) + threadIdx.x;
        }
#pragma unroll
        for (int q = 0; q < IB; ++q) {
            const T *src = out + static_cast<int64_t>(e[q].y) * row_elems;
#pragma unroll
            for (int k = 0; k < UNROLL; ++k) {
                const int64_t i = base[q] + k * 256;
                if (e[q].x >= 0 && i < row_elems) v[q][k] = (e[q].y >= 0) ? src[i] : T{};
            }
        }
#pragma unroll
        for (int q = 0; q < IB; ++q) {
            T *dst = out + static_cast<int64_t>(e[q].x) * row_elems;
#pragma unroll
            for (int k = 0; k < UNROLL; ++k) {
                const int64_t i = base[q] + k * 256;
                if (e[q].x >= 0 && i < row_elems) __builtin_nontemporal_store(v[q][k], dst + i);
            }
        }
    }
}

hipError_t launch_node_rows(const int32_t *unpacker, int B, int W, int L, int32_t *node_row, int2 *todo,
                            int32_t *ntodo, hipStream_t stream) {
    hipLaunchKernelGGL(k_node_rows, dim3(B), dim3(256), 0, stream, unpacker, W, L, node_row, todo, ntodo);
    return hipGetLastError();
}

hipError_t launch_unpack_dups(void *unpacked, const int2 *todo, const int32_t *ntodo, int64_t row_bytes, int B,
                              int W, int L, hipStream_t stream) {
    // workgroups per request: enough to spread a long list over the CUs
    constexpr int S = 32;
    constexpr int U = 4;
    auto go = [&](auto *dst, int64_t elems) {
        using T = std::remove_pointer_t<decltype(dst)>;
        const int nchunks = static_cast<int>((elems + 256 * U - 1) / (256 * U));
        hipLaunchKernelGGL((k_unpack_dups<T, U, 4>), dim3(static_cast<unsigned>(B * S)), dim3(256), 0, stream, dst,
                           todo, ntodo, elems, W * L, nchunks, S);
    };
    const uintptr_t align = reinterpret_cast<uintptr_t>(unpacked);
    if (row_bytes % 16 == 0 && align % 16 == 0)
        go(static_cast<u32x4 *>(unpacked), row_bytes / 16);
    else if (row_bytes % 4 == 0 && align % 4 == 0)
        go(static_cast<uint32_t *>(unpacked), row_bytes / 4);
    else
        go(static_cast<uint8_t *>(unpacked), row_bytes);
    return hipGetLastError();
}

hipError_t launch_unpack_accept(const void *packed, void *unpacked, const int32_t *unpacker, int64_t row_bytes,
                                const int32_t *beams, const int32_t *pargmax, int B, int W, int L,
                                int32_t *match_len, int32_t *best_beam, int32_t *accept_len,
                                int32_t *accepted, hipStream_t stream, const int32_t *bwid, const int32_t *blen) {
    AcceptArgs acc{beams, unpacker, pargmax, W, L, match_len, best_beam, accept_len, accepted, bwid, blen};
    if (!packed || !unpacked || row_bytes <= 0) {
        hipLaunchKernelGGL(k_accept, dim3(B), dim3(kWave), 0, stream, acc);
        return hipGetLastError();
    }
    const int64_t rows = static_cast<int64_t>(B) * W * L;
    const int P = W * L;
    const uintptr_t align = reinterpret_cast<uintptr_t>(packed) | reinterpret_cast<uintptr_t>(unpacked);
    constexpr int U = 4;
    auto go = [&](auto *src, auto *dst, int64_t elems) {
        using T = std::remove_const_t<std::remove_pointer_t<decltype(src)>>;
        const int nchunks = static_cast<int>((elems + 256 * U - 1) / (256 * U));
        const int64_t ncopy = rows * nchunks;
        hipLaunchKernelGGL((k_unpack_accept<T, U>), dim3(static_cast<unsigned>(ncopy + B)), dim3(256), 0, stream,
                           src, dst, unpacker, elems, P, W * L, nchunks, ncopy, acc);
    };
    if (row_bytes % 16 == 0 && align % 16 == 0)
        go(static_cast<const u32x4 *>(packed), static_cast<u32x4 *>(unpacked), row_bytes / 16);
    else if (row_bytes % 4 == 0 && align % 4 == 0)
        go(static_cast<const uint32_t *>(packed), static_cast<uint32_t *>(unpacked), row_bytes / 4);
    else
        go(static_cast<const uint8_t *>(packed), static_cast<uint8_t *>(unpacked), row_bytes);
    return hipGetLastError();
}

}  // namespace rd
