// Stochastic verification of the token tree by multi-step speculative
// sampling ("Accelerating LLM inference with speculative decoding" survey:
// rejection sampling keeps a draft x ~ q when u < p(x)/q(x); SpecInfer's
// random decoding applies that test to each drafted candidate in turn, and
// when all are rejected samples what remains of p, matching the target's
// sampling distribution).
//
// One 1024-thread workgroup per request walks the tree from slot 0.  At
// node u, p0 = softmax(logits[u]) is never stored: its max and sum are
// reduced once and p0(x) recomputed where needed.  All children of u share
// q = q[u], so the residual after i rejections has the closed form
// p_i = max(p0 - c_i q, 0) / D_i, with c_0 = 0, D_0 = 1 and, after a
// rejection, c <- c + D, D <- sum max(p0 - c q, 0) (kept when that sum is
// 0): by induction max(p_i - q, 0) = max(p0 - (c_i + D_i) q, 0) / D_i, the
// rows where p0 <= c_i q staying zero.  So a rejection costs one read-only
// reduction and no rewrite of a vector.  Children of u (slots whose parent
// is u, all above u) are found in slot order by a block-wide scan of a flag
// per slot; each is tested with u_accept * q(x) < p_i(x).  With no child
// accepted (or at a leaf) the bonus token is the first index whose running
// sum of max(p0 - c q, 0) exceeds u_bonus times its total: each thread sums
// a contiguous segment, one block scan orders the segments, and the thread
// whose segment holds the crossing finds it.  All sums run in a fixed
// order, so results are deterministic.
#include <math.h>

#include "rd_common.h"
#include "rd_internal.h"

namespace rd {

namespace {

constexpr int kT = 1024;              // threads per workgroup
constexpr int kNW = kT / kWave;       // wavefronts
constexpr int kMaxSlots = kMaxBeams * kMaxBeamLen;

struct StochArgs {
    const int32_t *unpacker, *plen, *ptok;
    const void *logits;  // [B,P,V] bf16 or f32
    const float *q;      // [B,P,V]
    const float *u_acc;  // [B,L,W]
    const float *u_bonus;
    int W, L, V, is_bf16;
    int32_t *best_beam, *accept_len, *accepted, *path;
};

__device__ __forceinline__ float load_logit(const StochArgs &a, size_t i) {
    if (a.is_bf16) {
        const uint16_t h = static_cast<const uint16_t *>(a.logits)[i];
        return __uint_as_float(static_cast<uint32_t>(h) << 16);
    }
    return static_cast<const float *>(a.logits)[i];
}

// Block reductions (fixed order: lanes by xor shuffles, then wavefronts in
// index order).  red is LDS scratch of kNW floats.
__device__ __forceinline__ float block_sum(float v, float *red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += shfl_xor(v, off);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) t += red[w];
    return t;
}

__device__ __forceinline__ float block_max(float v, float *red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, shfl_xor(v, off));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) t = fmaxf(t, red[w]);
    return t;
}

// Inclusive block scan of one float per thread; returns the thread's
// inclusive prefix and the block total.
__device__ __forceinline__ float block_scan(float v, float *red, float &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    __syncthreads();
    if (lane == 63) red[wave] = v;
    __syncthreads();
    float before = 0.f, t = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
        if (w < wave) before += red[w];
        t += red[w];
    }
    total = t;
    return before + v;
}

__device__ __forceinline__ int block_count_scan(int flag, int *redi, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t bal = __ballot(flag);
    const int below = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    __syncthreads();
    if (lane == 0) redi[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, t = 0;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
        if (w < wave) before += redi[w];
        t += redi[w];
    }
    total = t;
    return before + below;  // exclusive rank of this thread's flag
}

// Visits x = tid, tid + kT, ... < V in batches of kUB, loads first (indices
// clamped into the row, so the loads issue together), then f(x, logit, q)
// for the valid ones.
constexpr int kUB = 16;  // loads in flight per thread per batch (a 32000 row: two round trips per pass)
template <typename F>
__device__ __forceinline__ void row_pass(const StochArgs &a, size_t lrow, const float *qrow, int V, F f) {
    for (int base = threadIdx.x; base < V; base += kT * kUB) {
        float lv[kUB], qv[kUB];
#pragma unroll
        for (int j = 0; j < kUB; ++j) {
            const int x = min(base + j * kT, V - 1);
            lv[j] = load_logit(a, lrow + x);
            qv[j] = qrow ? qrow[x] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kUB; ++j)
            if (base + j * kT < V) f(base + j * kT, lv[j], qv[j]);
    }
}

__global__ __launch_bounds__(kT) void k_stochastic_accept(StochArgs a) {
    __shared__ int parent[kMaxSlots];
    __shared__ int kids[kMaxBeams];
    __shared__ float red[kNW];
    __shared__ int redi[kNW];
    __shared__ int nkids_sh;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int W = a.W, L = a.L, V = a.V;
    const int P = W * L;
    const int n = min(max(a.plen[b], 0), P);
    int32_t *acc_row = a.accepted + static_cast<size_t>(b) * L;
    int32_t *path_row = a.path ? a.path + static_cast<size_t>(b) * L : nullptr;
    for (int i = tid; i < L; i += kT) {
        acc_row[i] = -1;
        if (path_row) path_row[i] = -1;
    }
    if (n == 0) {
        if (tid == 0) {
            a.best_beam[b] = -1;
            a.accept_len[b] = -1;
        }
        return;
    }
    // parent of every slot (the same for every candidate that maps to it)
    const int32_t *un = a.unpacker + static_cast<size_t>(b) * P;
    for (int i = tid; i < P; i += kT) parent[i] = -1;
    __syncthreads();
    for (int i = tid; i < P; i += kT) {
        const int l = i % L;
        const int c = un[i];
        if (l > 0 && c >= 0 && c < n) parent[c] = un[i - 1];
    }
    __syncthreads();

    const size_t ubase = static_cast<size_t>(b) * P;
    int u = 0, d = 0, nacc = 0;
    float M = 0.f, invS = 1.f, c = 0.f;  // p0 = exp(l - M) * invS at node u; residual offset c
    size_t lrow = 0;
    const float *qrow = nullptr;
    auto p0v = [&](float l) { return __expf(l - M) * invS; };
    if (tid == 0 && path_row) path_row[0] = 0;
    while (true) {
        lrow = (ubase + u) * static_cast<size_t>(V);
        qrow = a.q + (ubase + u) * static_cast<size_t>(V);
        float m = -INFINITY;
        row_pass(a, lrow, nullptr, V, [&](int, float l, float) { m = fmaxf(m, l); });
        M = block_max(m, red);
        float s = 0.f;
        row_pass(a, lrow, nullptr, V, [&](int, float l, float) { s += __expf(l - M); });
        invS = 1.f / block_sum(s, red);
        c = 0.f;
        float D = 1.f;
        // children of u in slot order
        int nk;
        {
            const int cs = tid;
            const int flag = (cs > u && cs < n && parent[cs] == u) ? 1 : 0;
            int tot;
            const int r = block_count_scan(flag, redi, tot);
            if (flag && r < kMaxBeams) kids[r] = cs;
            if (tid == 0) nkids_sh = min(tot, kMaxBeams);
            __syncthreads();
            nk = nkids_sh;
        }
        int next = -1;
        for (int i = 0; i < nk; ++i) {
            const int ch = kids[i];
            const int x = min(max(a.ptok[ubase + ch], 0), V - 1);
            const float r = a.u_acc[(static_cast<size_t>(b) * L + d) * W + min(i, W - 1)];
            const float px = fmaxf(p0v(load_logit(a, lrow + x)) - c * qrow[x], 0.f) / D;
            if (r * qrow[x] < px) {  // the same values in every thread: a uniform branch
                next = ch;
                break;
            }
            const float cn = c + D;
            float t = 0.f;
            row_pass(a, lrow, qrow, V, [&](int, float l, float qv) { t += fmaxf(p0v(l) - cn * qv, 0.f); });
            const float T = block_sum(t, red);
            if (T > 0.f) {
                c = cn;
                D = T;
            }
        }
        if (next < 0) break;
        if (tid == 0) {
            acc_row[nacc] = a.ptok[ubase + next];
            if (path_row) path_row[d + 1] = next;
        }
        u = next;
        ++d;
        ++nacc;
    }
    // bonus: first index whose running sum of max(p0 - c q, 0) exceeds
    // u_bonus times the total; thread t owns the contiguous segment
    // [t*seg, (t+1)*seg)
    const int seg = (V + kT - 1) / kT;
    const int x0 = min(tid * seg, V), x1 = min(x0 + seg, V);
    // weights of a batch of the thread's segment (loads issued together)
    auto seg_batch = [&](int xb, float (&wv)[kUB]) {
        float lv[kUB], qv[kUB];
#pragma unroll
        for (int j = 0; j < kUB; ++j) {
            const int x = min(xb + j, x1 - 1);
            lv[j] = load_logit(a, lrow + x);
            qv[j] = qrow[x];
        }
#pragma unroll
        for (int j = 0; j < kUB; ++j) wv[j] = (xb + j < x1) ? fmaxf(p0v(lv[j]) - c * qv[j], 0.f) : 0.f;
    };
    float part = 0.f;
    for (int xb = x0; xb < x1; xb += kUB) {
        float wv[kUB];
        seg_batch(xb, wv);
#pragma unroll
        for (int j = 0; j < kUB; ++j) part += wv[j];
    }
    float total;
    const float exc = block_scan(part, red, total) - part;
    const float thr = a.u_bonus[b] * total;
    // a segment whose running sum already exceeds the threshold at its start
    // proposes its first index, so rounding between segments cannot hide the
    // crossing; the lowest proposal wins
    int cand = V;
    if (x0 < x1) {
        if (exc > thr) {
            cand = x0;
        } else {
            float acc = exc;
            for (int xb = x0; xb < x1 && cand == V; xb += kUB) {
                float wv[kUB];
                seg_batch(xb, wv);
#pragma unroll
                for (int j = 0; j < kUB; ++j) {
                    acc += wv[j];
                    if (cand == V && xb + j < x1 && acc > thr) cand = xb + j;
                }
            }
        }
    }
    // lowest candidate over the workgroup
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cand = min(cand, __shfl_xor(cand, off, 64));
    __syncthreads();
    if ((tid & 63) == 0) redi[tid >> 6] = cand;
    __syncthreads();
    if (tid == 0) {
        int bonus = V;
        for (int w = 0; w < kNW; ++w) bonus = min(bonus, redi[w]);
        acc_row[nacc] = min(bonus, V - 1);
        a.accept_len[b] = nacc;
        int best = -1;
        for (int w = 0; w < W && best < 0; ++w)
            if (un[w * L + nacc] == u) best = w;
        a.best_beam[b] = best;
    }
}

}  // namespace

hipError_t launch_stochastic_accept(int dtype, const int32_t *unpacker, const int32_t *plen, const int32_t *ptok,
                                    const void *logits, const float *q, const float *u_accept, const float *u_bonus,
                                    int B, int W, int L, int V, int32_t *best_beam, int32_t *accept_len,
                                    int32_t *accepted, int32_t *path, hipStream_t stream) {
    StochArgs a{unpacker, plen, ptok, logits, q, u_accept, u_bonus, W, L, V, dtype == 1 ? 1 : 0,
                best_beam, accept_len, accepted, path};
    hipLaunchKernelGGL(k_stochastic_accept, dim3(B), dim3(kT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rd
