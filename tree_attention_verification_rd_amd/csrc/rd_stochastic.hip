// Stochastic verification of the token tree by multi-step speculative
// sampling ("Accelerating LLM inference with speculative decoding" survey:
// rejection sampling keeps a draft x ~ q when u < p(x)/q(x); SpecInfer's
// random decoding applies that test to each drafted candidate in turn, and
// when all are rejected samples what remains of p, matching the target's
// sampling distribution).
//
// p0 = softmax(logits[u]) is never stored: its max and sum are reduced and
// p0(x) recomputed where needed.  All children of node u share q = q[u], so
// the residual after i rejections has the closed form
// p_i = max(p0 - c_i q, 0) / D_i, with c_0 = 0, D_0 = 1 and, after a
// rejection, c <- c + D, D <- sum max(p0 - c q, 0) (kept when that sum is
// 0): by induction max(p_i - q, 0) = max(p0 - (c_i + D_i) q, 0) / D_i, the
// rows where p0 <= c_i q staying zero.  The sequence (c_i, D_i) of a node
// depends on its p0 and q only, not on the uniforms, so it is computed for
// every node at once:
//   k_stoch_rows  -- bf16 logits, V a multiple of 8 and at most 32768 (the
//                    rows the workloads have): the statistics listed next,
//                    in persistent workgroups of 512 threads that hold a row
//                    in registers (64 entries a thread) and load the next
//                    slot's row while computing the current one (see there);
//   k_stoch_node  -- otherwise, one workgroup per (request, slot): the max and sum of
//                    the slot's logits, (c_i, D_i) for i up to its child
//                    count nk, the pair (p_i(x), q(x)) that its i-th child
//                    (token x) is tested with, stored with that child, and
//                    the bonus token the slot yields if every child is
//                    rejected: the first index whose running sum of
//                    w = max(p0 - c_nk q, 0) exceeds u_bonus times its total.
//                    Up to 32K entries the row stays in registers (thread t
//                    holds groups of 8 consecutive entries x = 8(t + 1024 g)
//                    + e, g < 4, loaded 16 bytes at a time when V is a
//                    multiple of 8); the four groups' sums pick the group
//                    holding the crossing, a block scan of the threads' sums
//                    there picks the thread, and its 8 entries the index.  Longer rows are streamed.  When V is
//                    a multiple of 8, every pass reads 16-byte groups of 8
//                    entries over one contiguous range per wave, so each
//                    pass also gives per-wave weight sums; the bonus then
//                    rescans only the range that holds the crossing.
//                    Otherwise entry by entry, each wave taking a contiguous
//                    range for the bonus;
//   k_stoch_walk  -- one workgroup per request: the pairs and the request's
//                    uniforms are staged in LDS; then wavefront 0, from slot 0: children
//                    (slots whose parent is the node, all above it) are
//                    found in slot order by ballots over 64 slots at a time
//                    and the i-th is accepted when u_accept * q(x) <
//                    p_i(x); the node where every child is rejected (or a
//                    leaf) gives its precomputed bonus.
// Every block of the grid does the work of one row, so the chip's
// bandwidth, not one CU's, bounds the pass over the logits.
// All sums run in a fixed order, so results are deterministic.
#include <math.h>

#include <algorithm>

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
    int B, W, L, V, is_bf16;
    int32_t *best_beam, *accept_len, *accepted, *path;
    float2 *test;    // [B,P]: (p_i(x), q(x)) of the slot's test at its parent (x its token, i its rank)
    int32_t *bonus;  // [B,P]: the slot's bonus token when all its children are rejected
};

__device__ __forceinline__ float load_logit(const StochArgs &a, size_t i) {
    if (a.is_bf16) {
        const uint16_t h = static_cast<const uint16_t *>(a.logits)[i];
        return __uint_as_float(static_cast<uint32_t>(h) << 16);
    }
    return static_cast<const float *>(a.logits)[i];
}

// Sum or maximum over the 64 lanes of a wavefront, the same bits in every
// lane, without LDS round trips: lanes i and i^32 by v_permlane32_swap, i
// and i^16 by v_permlane16_swap (with both operands v each leaves the two
// lanes' values in its two results), then within each row of 16 lanes DPP
// rotations by 8, 4, 2 and 1.  Each step combines two equal partial results
// with a commutative operation, so all lanes agree.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    v = op(v, dpp_f<0x128>(v));  // row_ror:8
    v = op(v, dpp_f<0x124>(v));  // row_ror:4
    v = op(v, dpp_f<0x122>(v));  // row_ror:2
    v = op(v, dpp_f<0x121>(v));  // row_ror:1
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce(v, [](float x, float y) { return x + y; });
}
__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}

// Block reductions (fixed order: the wavefront's lanes as above, then
// wavefronts in index order).  red is LDS scratch of kNW floats.
template <int NT = kT>
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < (NT / kWave); ++w) t += red[w];
    return t;
}

template <int NT = kT>
__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = -INFINITY;
#pragma unroll
    for (int w = 0; w < (NT / kWave); ++w) t = fmaxf(t, red[w]);
    return t;
}

// (max, sum of exp(l - max)) of the block from each thread's pair (online
// softmax: two pairs merge as M = max, s = s1 e^(m1-M) + s2 e^(m2-M)).
// red is LDS scratch of 2 kNW floats.  Returns M; S in *S.
__device__ __forceinline__ float merge_scale(float m, float M) { return m == -INFINITY ? 0.f : __expf(m - M); }
template <int NT = kT>
__device__ __forceinline__ float block_softmax_stats(float m, float s, float *red, float *S) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float mo = shfl_xor(m, off), so = shfl_xor(s, off);
        const float M = fmaxf(m, mo);
        s = s * merge_scale(m, M) + so * merge_scale(mo, M);
        m = M;
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        red[threadIdx.x >> 6] = m;
        red[(NT / kWave) + (threadIdx.x >> 6)] = s;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < (NT / kWave); ++w) M = fmaxf(M, red[w]);
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < (NT / kWave); ++w) t += red[(NT / kWave) + w] * merge_scale(red[w], M);
    *S = t;
    return M;
}

// Inclusive block scan of one float per thread; returns the thread's
// inclusive prefix and the block total.
// Inclusive scan over the lanes of a wavefront, without LDS round trips:
// shifts by 1, 2, 4 and 8 within each row of 16 lanes (lanes shifted in from
// outside the row read 0), then the last lane of row 0 (2) added to row 1
// (3), then the last lane of row 1 to rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f0(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, true));
}
__device__ __forceinline__ float wave_scan_incl(float v) {
    v += dpp_f0<0x111, 0xF>(v);  // row_shr:1
    v += dpp_f0<0x112, 0xF>(v);  // row_shr:2
    v += dpp_f0<0x114, 0xF>(v);  // row_shr:4
    v += dpp_f0<0x118, 0xF>(v);  // row_shr:8
    v += dpp_f0<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_f0<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

template <int NT = kT>
__device__ __forceinline__ float block_scan(float v, float *red, float &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_scan_incl(v);
    __syncthreads();
    if (lane == 63) red[wave] = v;
    __syncthreads();
    float before = 0.f, t = 0.f;
#pragma unroll
    for (int w = 0; w < (NT / kWave); ++w) {
        if (w < wave) before += red[w];
        t += red[w];
    }
    total = t;
    return before + v;
}

template <int NT = kT>
__device__ __forceinline__ int block_count_scan(int flag, int *redi, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t bal = __ballot(flag);
    const int below = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    __syncthreads();
    if (lane == 0) redi[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, t = 0;
#pragma unroll
    for (int w = 0; w < (NT / kWave); ++w) {
        if (w < wave) before += redi[w];
        t += redi[w];
    }
    total = t;
    return before + below;  // exclusive rank of this thread's flag
}

// Inclusive block scan of one int per thread; total receives the block sum.
template <int NT = kT>
__device__ __forceinline__ int block_scan_int(int v, int *redi, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    __syncthreads();
    if (lane == 63) redi[wave] = v;
    __syncthreads();
    int before = 0, t = 0;
#pragma unroll
    for (int w = 0; w < (NT / kWave); ++w) {
        if (w < wave) before += redi[w];
        t += redi[w];
    }
    total = t;
    return before + v;
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

// This thread's RJ entries of a row: entry j is x = 8*(tid + kT*(j/8)) + j%8,
// so each group of 8 is consecutive.  When V is a multiple of 8 every group
// is one 16-byte load of bf16 logits (two of f32) and two of q; otherwise
// the same entries are loaded one by one.  Reads past the row give zero.
template <int NT = kT>
__device__ __forceinline__ int reg_x(int j) { return 8 * (static_cast<int>(threadIdx.x) + NT * (j >> 3)) + (j & 7); }
template <int RJ>
__device__ __forceinline__ void load_row_regs(const StochArgs &a, size_t lrow, float (&lv)[RJ], float (&qv)[RJ]) {
    static_assert(RJ % 8 == 0, "whole groups of 8 entries");
    constexpr int RG = RJ / 8;
    const uint32_t V = static_cast<uint32_t>(a.V), t = threadIdx.x;
    const rsrc_t rq = make_rsrc(a.q + lrow, V * 4u);
    if (V % 8 == 0) {
        u32x4 l0[RG], l1[RG], q0[RG], q1[RG];
        if (a.is_bf16) {
            const rsrc_t rl = make_rsrc(static_cast<const uint16_t *>(a.logits) + lrow, V * 2u);
#pragma unroll
            for (int g = 0; g < RG; ++g) l0[g] = __builtin_amdgcn_raw_buffer_load_b128(rl, (t + kT * g) * 16u, 0, 0);
        } else {
            const rsrc_t rl = make_rsrc(static_cast<const float *>(a.logits) + lrow, V * 4u);
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                l0[g] = __builtin_amdgcn_raw_buffer_load_b128(rl, (t + kT * g) * 32u, 0, 0);
                l1[g] = __builtin_amdgcn_raw_buffer_load_b128(rl, (t + kT * g) * 32u + 16u, 0, 0);
            }
        }
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            q0[g] = __builtin_amdgcn_raw_buffer_load_b128(rq, (t + kT * g) * 32u, 0, 0);
            q1[g] = __builtin_amdgcn_raw_buffer_load_b128(rq, (t + kT * g) * 32u + 16u, 0, 0);
        }
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (a.is_bf16) {
                    lv[8 * g + 2 * k] = __uint_as_float(l0[g][k] << 16);
                    lv[8 * g + 2 * k + 1] = __uint_as_float(l0[g][k] & 0xFFFF0000u);
                } else {
                    lv[8 * g + k] = __uint_as_float(l0[g][k]);
                    lv[8 * g + 4 + k] = __uint_as_float(l1[g][k]);
                }
                qv[8 * g + k] = __uint_as_float(q0[g][k]);
                qv[8 * g + 4 + k] = __uint_as_float(q1[g][k]);
            }
        return;
    }
    if (a.is_bf16) {
        const rsrc_t rl = make_rsrc(static_cast<const uint16_t *>(a.logits) + lrow, V * 2u);
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
            const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(rl, static_cast<uint32_t>(reg_x(j)) * 2u, 0, 0);
            lv[j] = __uint_as_float(h << 16);
        }
    } else {
        const rsrc_t rl = make_rsrc(static_cast<const float *>(a.logits) + lrow, V * 4u);
#pragma unroll
        for (int j = 0; j < RJ; ++j)
            lv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, static_cast<uint32_t>(reg_x(j)) * 4u, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < RJ; ++j)
        qv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rq, static_cast<uint32_t>(reg_x(j)) * 4u, 0, 0));
}

// Rows whose length is a multiple of 8 are streamed with 16-byte loads:
// group g holds entries 8g .. 8g+7 (one dwordx4 of bf16 logits or two of
// f32, two of q).  Offsets past the row read as zero and are masked by the
// callers.  One wave-wide load then moves 1 KB instead of 128-256 bytes, so a
// pass over a long row is no longer bound by the rate at which the CU
// accepts load instructions.
struct RowRes {
    rsrc_t l, q;
};
__device__ __forceinline__ RowRes row_res(const StochArgs &a, size_t lrow) {
    const uint32_t V = static_cast<uint32_t>(a.V);
    RowRes r;
    r.l = a.is_bf16 ? make_rsrc(static_cast<const uint16_t *>(a.logits) + lrow, V * 2u)
                    : make_rsrc(static_cast<const float *>(a.logits) + lrow, V * 4u);
    r.q = make_rsrc(a.q + lrow, V * 4u);
    return r;
}
struct Grp {
    u32x4 l0, l1, q0, q1;
};
__device__ __forceinline__ Grp load_grp(const StochArgs &a, const RowRes &r, uint32_t g, bool with_q) {
    Grp v;
    if (a.is_bf16) {
        v.l0 = __builtin_amdgcn_raw_buffer_load_b128(r.l, g * 16u, 0, 0);
        v.l1 = u32x4{0, 0, 0, 0};
    } else {
        v.l0 = __builtin_amdgcn_raw_buffer_load_b128(r.l, g * 32u, 0, 0);
        v.l1 = __builtin_amdgcn_raw_buffer_load_b128(r.l, g * 32u + 16u, 0, 0);
    }
    if (with_q) {
        v.q0 = __builtin_amdgcn_raw_buffer_load_b128(r.q, g * 32u, 0, 0);
        v.q1 = __builtin_amdgcn_raw_buffer_load_b128(r.q, g * 32u + 16u, 0, 0);
    } else {
        v.q0 = v.q1 = u32x4{0, 0, 0, 0};
    }
    return v;
}
// entries of a loaded group as floats, in index order
__device__ __forceinline__ void unpack_grp(const StochArgs &a, const Grp &v, float (&l)[8], float (&q)[8]) {
    if (a.is_bf16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            l[2 * k] = __uint_as_float(v.l0[k] << 16);
            l[2 * k + 1] = __uint_as_float(v.l0[k] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            l[k] = __uint_as_float(v.l0[k]);
            l[4 + k] = __uint_as_float(v.l1[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        q[k] = __uint_as_float(v.q0[k]);
        q[4 + k] = __uint_as_float(v.q1[k]);
    }
}

// Groups of a row are split into kNW contiguous ranges, one per wavefront
// (the same ranges in every pass, so each pass also yields per-wavefront
// sums).  A wavefront walks its range 64 groups (1 KB of bf16 logits) a
// step, kSBV steps loaded together, calling f(l[8], q[8]) on each group.
constexpr int kSBV = 4;
template <int NT = kT>
__device__ __forceinline__ void wave_range(int G, int &g0, int &g1) {
    const int GW = (G + (NT / kWave) - 1) / (NT / kWave);
    g0 = min(static_cast<int>(threadIdx.x >> 6) * GW, G);
    g1 = min(g0 + GW, G);
}
template <typename F>
__device__ __forceinline__ void wave_pass(const StochArgs &a, const RowRes &r, bool with_q, int g0, int g1, F f) {
    const int lane = threadIdx.x & 63;
    for (int s0 = 0; s0 < g1 - g0; s0 += 64 * kSBV) {
        Grp v[kSBV];
#pragma unroll
        for (int j = 0; j < kSBV; ++j) v[j] = load_grp(a, r, static_cast<uint32_t>(g0 + s0 + 64 * j + lane), with_q);
#pragma unroll
        for (int j = 0; j < kSBV; ++j)
            if (g0 + s0 + 64 * j + lane < g1) {
                float l[8], q[8];
                unpack_grp(a, v[j], l, q);
                f(l, q);
            }
    }
}

// parent slot of every slot of request b (-1 for roots), into LDS
template <int NT = kT>
__device__ __forceinline__ void build_parents(const StochArgs &a, int b, int n, int *parent) {
    const int P = a.W * a.L;
    const int32_t *un = a.unpacker + static_cast<size_t>(b) * P;
    for (int i = threadIdx.x; i < P; i += NT) parent[i] = -1;
    __syncthreads();
    for (int i = threadIdx.x; i < P; i += NT) {
        const int l = i % a.L;
        const int c = un[i];
        if (l > 0 && c >= 0 && c < n) parent[c] = un[i - 1];
    }
    __syncthreads();
}

// children of slot u in slot order into kids (at most kMaxBeams); returns their count
template <int NT = kT>
__device__ __forceinline__ int children_of(int u, int n, const int *parent, int *kids, int *redi, int *cnt_sh) {
    int carry = 0;
    for (int c0 = 0; c0 < n; c0 += NT) {
        const int cs = c0 + static_cast<int>(threadIdx.x);
        const int flag = (cs > u && cs < n && parent[cs] == u) ? 1 : 0;
        int tot;
        const int r = carry + block_count_scan<NT>(flag, redi, tot);
        if (flag && r < kMaxBeams) kids[r] = cs;
        carry += tot;
    }
    if (threadIdx.x == 0) *cnt_sh = min(carry, kMaxBeams);
    __syncthreads();
    return *cnt_sh;
}

// Bonus of a register-resident row: thread t holds p0 and q of its entries
// x = reg_x(j) in pv[j], qv[j] (zeros past the row), so the weight of x is
// max(pv[j] - c qv[j], 0).  The row is RJ/8 groups of 8*NT consecutive
// entries.  The group holding the crossing of u_b times the total is found
// from the groups' sums, then the thread by a block scan of the threads' sums
// in that group, then the entry among the thread's 8.  When rounding between
// the levels hides the crossing, the last entry of nonzero weight of the
// chosen group (or thread) stands in, where the crossing lies in exact
// arithmetic.  Returns the index in every thread.
// With have, tsk holds this thread's group sums of the weights for this c
// already (from the residual pass that set c); otherwise they are formed
// here.  gsum is 16-byte aligned.
template <int RJ, int NT = kT>
__device__ __forceinline__ int bonus_regs(const float (&pv)[RJ], const float (&qv)[RJ], float c, float u_b,
                                          float *red, int *redi, float *gsum, const float (&tsk)[RJ / 8],
                                          bool have) {
    constexpr int RG = RJ / 8;
    constexpr int NW = NT / kWave;
    static_assert(NW % 4 == 0, "group sums are read four at a time");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // weights are recomputed where needed rather than held (registers)
    auto w = [&](int j) { return fmaxf(pv[j] - c * qv[j], 0.f); };
    float ts[RG];  // this thread's sum in each group
    if (have) {
#pragma unroll
        for (int g = 0; g < RG; ++g) ts[g] = tsk[g];
    } else {
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            ts[g] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ts[g] += w(8 * g + e);
        }
    }
    // group sums: per wave, then the waves in index order
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const float v = wave_sum(ts[g]);
        if (lane == 0) gsum[g * (NT / kWave) + wave] = v;
    }
    __syncthreads();
    float S[RG], total = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        S[g] = 0.f;
#pragma unroll
        for (int w4 = 0; w4 < NW / 4; ++w4) {
            const float4 f = *reinterpret_cast<const float4 *>(gsum + g * NW + 4 * w4);
            S[g] += f.x;
            S[g] += f.y;
            S[g] += f.z;
            S[g] += f.w;
        }
        total += S[g];
    }
    const float thr = u_b * total;
    int gs = -1, glast = 0;
    float E = 0.f, run = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        if (gs < 0 && run + S[g] > thr) {
            gs = g;
            E = run;
        }
        if (S[g] > 0.f) glast = g;
        run += S[g];
    }
    const bool exact = gs >= 0;
    if (!exact) gs = glast;
    float mine = 0.f;  // this thread's sum in the chosen group
#pragma unroll
    for (int g = 0; g < RG; ++g)
        if (g == gs) mine = ts[g];
    float tot;
    const float inc = block_scan<NT>(mine, red, tot);
    const uint64_t hit = __ballot(exact && E + inc > thr);
    const uint64_t nz = __ballot(mine > 0.f);
    if (lane == 0) {
        redi[wave] = hit ? wave * 64 + __ffsll(static_cast<long long>(hit)) - 1 : NT;
        redi[(NT / kWave) + wave] = nz ? wave * 64 + 63 - __clzll(static_cast<long long>(nz)) : -1;
    }
    __syncthreads();
    int first = NT, last = -1;
#pragma unroll
    for (int w2 = 0; w2 < (NT / kWave); ++w2) {
        first = min(first, redi[w2]);
        last = max(last, redi[(NT / kWave) + w2]);
    }
    const int tsel = first < NT ? first : max(last, 0);
    // the entry among the chosen thread's 8 (its running sum from E + its exclusive prefix)
    if (static_cast<int>(threadIdx.x) == tsel) {
        // the same weights again, from a copy of c the compiler cannot see
        // through: merged with the ones summed above, all RJ would be held
        // across the block scan
        float c2 = c;
        asm volatile("" : "+v"(c2));
        auto w2 = [&](int j) { return fmaxf(pv[j] - c2 * qv[j], 0.f); };
        float r = E + (inc - mine);
        int es = -1, enz = 0;
#pragma unroll
        for (int g = 0; g < RG; ++g)
            if (g == gs) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float we = w2(8 * g + e);
                    r += we;
                    if (es < 0 && first < NT && r > thr) es = e;
                    if (we > 0.f) enz = e;
                }
            }
        redi[2 * (NT / kWave)] = 8 * (tsel + NT * gs) + (es >= 0 ? es : enz);
    }
    __syncthreads();
    return redi[2 * (NT / kWave)];
}

template <int RJ, int NT = kT>
__device__ __forceinline__ int bonus_regs(const float (&pv)[RJ], const float (&qv)[RJ], float c, float u_b,
                                          float *red, int *redi, float *gsum) {
    const float none[RJ / 8] = {};
    return bonus_regs<RJ, NT>(pv, qv, c, u_b, red, redi, gsum, none, false);
}

// Bonus of a streamed row (p0 = exp(l - M) * invS, weight max(p0 - c q, 0)):
// wave wv owns the contiguous range [wv*RW, (wv+1)*RW) and reads it 64
// entries a step.  A range whose running sum already exceeds the threshold at
// its start proposes its first index, so rounding between ranges cannot hide
// the crossing; the lowest proposal wins, and with none the last index of
// nonzero weight stands in.  Result valid in every thread.
__device__ __forceinline__ int bonus_streamed(const StochArgs &a, size_t lrow, const float *qrow, float M, float invS,
                                              float c, float u_b, float *red, int *redi) {
    const int V = a.V;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int RW = (V + kNW - 1) / kNW;
    const int r0 = min(wv * RW, V), r1 = min(r0 + RW, V);
    const int nsteps = (r1 - r0 + 63) / 64;
    constexpr int kSB = 16;  // steps loaded together
    auto step_weights = [&](int s0, float (&w)[kSB]) {
        float lv[kSB], qv[kSB];
#pragma unroll
        for (int j = 0; j < kSB; ++j) {
            const int x = min(r0 + (s0 + j) * 64 + lane, max(r1 - 1, 0));
            lv[j] = load_logit(a, lrow + x);
            qv[j] = qrow[x];
        }
#pragma unroll
        for (int j = 0; j < kSB; ++j)
            w[j] = (r0 + (s0 + j) * 64 + lane < r1) ? fmaxf(__expf(lv[j] - M) * invS - c * qv[j], 0.f) : 0.f;
    };
    float lsum = 0.f;
    int lastnz = -1;
    for (int s0 = 0; s0 < nsteps; s0 += kSB) {
        float w[kSB];
        step_weights(s0, w);
#pragma unroll
        for (int j = 0; j < kSB; ++j) {
            lsum += w[j];
            if (w[j] > 0.f) lastnz = r0 + (s0 + j) * 64 + lane;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        lsum += shfl_xor(lsum, off);  // the wave's total, in every lane
        lastnz = max(lastnz, shfl_xor(lastnz, off));
    }
    __syncthreads();
    if (lane == 0) {
        red[wv] = lsum;
        redi[kNW + wv] = lastnz;
    }
    __syncthreads();
    float exc = 0.f, total = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kNW; ++w2) {
        if (w2 < wv) exc += red[w2];
        total += red[w2];
    }
    const float thr = u_b * total;
    int cand = V;
    if (r0 < r1) {
        if (exc > thr) {
            cand = r0;
        } else {
            float carry = exc;
            for (int s0 = 0; s0 < nsteps && cand == V; s0 += kSB) {
                float w[kSB];
                step_weights(s0, w);
#pragma unroll
                for (int j = 0; j < kSB; ++j) {
                    float inc = w[j];
#pragma unroll
                    for (int off = 1; off < 64; off <<= 1) {
                        const float o = __shfl_up(inc, off, 64);
                        if (lane >= off) inc += o;
                    }
                    const float tot = __shfl(inc, 63, 64);
                    const uint64_t hit = __ballot(carry + inc > thr && r0 + (s0 + j) * 64 + lane < r1);
                    if (cand == V && hit) cand = r0 + (s0 + j) * 64 + __ffsll(static_cast<long long>(hit)) - 1;
                    carry += tot;
                }
            }
        }
    }
    if (lane == 0) redi[wv] = cand;
    __syncthreads();
    int first = V, last = 0;
#pragma unroll
    for (int w2 = 0; w2 < kNW; ++w2) {
        first = min(first, redi[w2]);
        last = max(last, redi[kNW + w2]);
    }
    return first < V ? first : last;
}

// Bonus of a row of V % 8 == 0 entries streamed in wavefront ranges.
// wtot[w] holds the sum of the weights w(x) = max(p0(x) - c q(x), 0) over
// wavefront w's range, from the pass that last set c.  The crossing lies in
// the first range whose running total exceeds u_b times the whole (with
// none, from rounding, the last range of nonzero total), and only that
// range is scanned: lane sums scanned across the wavefront, then the 8
// entries of the crossing lane.  Where rounding between the levels hides
// the crossing, the range's last entry of nonzero weight stands in.  Result
// valid in every thread.
template <int NT = kT>
__device__ __forceinline__ int bonus_streamed_vec(const StochArgs &a, const RowRes &r, float M, float invS, float c,
                                                  float u_b, const float *wtot, int *redi) {
    const int V = a.V;
    const int G = V / 8;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    float total = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < (NT / kWave); ++w2) total += wtot[w2];
    const float thr = u_b * total;
    int ws = -1, wlast = -1;
    float exc = 0.f, ews = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < (NT / kWave); ++w2) {
        if (ws < 0 && exc + wtot[w2] > thr) {
            ws = w2;
            ews = exc;
        }
        if (wtot[w2] > 0.f) wlast = w2;
        exc += wtot[w2];
    }
    if (ws < 0) {  // rounding put the threshold at or past the total
        ws = wlast >= 0 ? wlast : (NT / kWave) - 1;
        ews = -INFINITY;  // never crosses: the range's last nonzero entry stands in
    }
    if (wv == ws) {
        int g0, g1;
        wave_range<NT>(G, g0, g1);
        int cand = -1, lastnz = -1;
        float carry = ews;
        for (int s0 = 0; s0 < g1 - g0 && cand < 0; s0 += 64 * kSBV) {
            Grp v[kSBV];
#pragma unroll
            for (int j = 0; j < kSBV; ++j)
                v[j] = load_grp(a, r, static_cast<uint32_t>(g0 + s0 + 64 * j + lane), true);
#pragma unroll
            for (int j = 0; j < kSBV; ++j) {
                const int g = g0 + s0 + 64 * j + lane;
                float l[8], q[8], w[8];
                unpack_grp(a, v[j], l, q);
                float tl = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    w[e] = g < g1 ? fmaxf(__expf(l[e] - M) * invS - c * q[e], 0.f) : 0.f;
                    tl += w[e];
                    if (w[e] > 0.f) lastnz = 8 * g + e;
                }
                float inc = tl;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float o = __shfl_up(inc, off, 64);
                    if (lane >= off) inc += o;
                }
                const float tot = __shfl(inc, 63, 64);
                const uint64_t hit = __ballot(carry + inc > thr && g < g1);
                if (cand < 0 && hit) {
                    const int hl = __ffsll(static_cast<long long>(hit)) - 1;
                    float run = carry + (inc - tl);
                    int es = -1, enz = 7;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        run += w[e];
                        if (es < 0 && run > thr) es = e;
                        if (w[e] > 0.f) enz = e;
                    }
                    const int eh = __shfl(es >= 0 ? es : enz, hl, 64);
                    cand = 8 * (g0 + s0 + 64 * j + hl) + eh;
                }
                carry += tot;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) lastnz = max(lastnz, shfl_xor(lastnz, off));
        if (lane == 0) redi[0] = cand >= 0 ? cand : max(lastnz, 0);
    }
    __syncthreads();
    return redi[0];
}

// Every statistic of one slot: (max, 1/sum) of its logits, the residual
// sequence (c_i, D_i) for i up to its child count, each child's test pair
// and the slot's bonus.  With RJ > 0 (V <= kT * RJ) the slot's logits and q
// are loaded once into registers (element x = tid + kT*j) and every pass runs
// on them; with RJ == 0 each pass streams the row entry by entry, with
// RJ < 0 (V a multiple of 8) in 16-byte groups of 8 entries.
template <int RJ, int NT = kT>
__global__ __launch_bounds__(NT, kT / NT) void k_stoch_node(StochArgs a) {
    static_assert(NT == kT || RJ < 0, "only the streamed 16-byte path runs with other workgroup sizes");
    __shared__ int parent[kMaxSlots];
    __shared__ int kids[kMaxBeams];
    __shared__ float2 cd_sh[kMaxBeams];
    __shared__ float red[2 * (NT / kWave)];
    __shared__ int redi[2 * (NT / kWave) + 1];
    __shared__ int tok_sh[kMaxSlots];
    __shared__ __attribute__((aligned(16))) float gsum[(RJ > 0 ? RJ / 8 : 1) * (NT / kWave)];
    __shared__ int nkids_sh;
    __shared__ float wtot[(NT / kWave)];  // streamed rows: per-wavefront weight sums for the bonus
    const int W = a.W, L = a.L, V = a.V;
    const int P = W * L;
    const int b = blockIdx.x / P;
    const int u = blockIdx.x % P;
    const int n = min(max(a.plen[b], 0), P);
    if (u >= n) return;
    const size_t ubase = static_cast<size_t>(b) * P;
    const size_t lrow = (ubase + u) * static_cast<size_t>(V);
    const float *qrow = a.q + lrow;
    const RowRes rr = row_res(a, lrow);
    int vg0 = 0, vg1 = 0;  // this wavefront's range of 8-entry groups (streamed rows)
    if constexpr (RJ < 0) wave_range<NT>(V / 8, vg0, vg1);
    float pv[RJ > 0 ? RJ : 1], qv[RJ > 0 ? RJ : 1];  // logits, then p0, and q of this thread's elements
    if constexpr (RJ > 0) load_row_regs<RJ>(a, lrow, pv, qv);  // issued first: the loads overlap the tree build
    for (int i = threadIdx.x; i < n; i += NT) tok_sh[i] = a.ptok[ubase + i];
    build_parents<NT>(a, b, n, parent);  // its barriers also publish tok_sh
    const int nk = children_of<NT>(u, n, parent, kids, redi, &nkids_sh);
    // thread i < nk: child i's token, its logit and q (their latency hides
    // behind the softmax statistics)
    int kid = -1;
    float kl = 0.f, kq = 0.f;
    if (static_cast<int>(threadIdx.x) < nk) {
        kid = kids[threadIdx.x];
        const int x = min(max(tok_sh[kid], 0), V - 1);
        kl = load_logit(a, lrow + x);
        kq = qrow[x];
    }
    // softmax statistics: from registers, the block max then the sum of
    // exp(l - M) (one exponential per entry); streamed, one pass of per-thread
    // (max, sum) pairs merged across the block
    float M, invS;
    if constexpr (RJ > 0) {
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < RJ; ++j)
            if (reg_x(j) < V) m = fmaxf(m, pv[j]);
        M = block_max(m, red);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
            const bool ok = reg_x(j) < V;
            pv[j] = ok ? __expf(pv[j] - M) : 0.f;
            qv[j] = ok ? qv[j] : 0.f;
            s += pv[j];
        }
        invS = 1.f / block_sum(s, red);
#pragma unroll
        for (int j = 0; j < RJ; ++j) pv[j] *= invS;
    } else if constexpr (RJ < 0) {
        // one rescale per group of 8: its max first, then the 8 exponentials
        float m = -INFINITY, s = 0.f;
        wave_pass(a, rr, false, vg0, vg1, [&](const float (&l)[8], const float (&)[8]) {
            float gm = l[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) gm = fmaxf(gm, l[e]);
            const float mn = fmaxf(m, gm);
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) t += __expf(l[e] - mn);
            s = s * merge_scale(m, mn) + t;
            m = mn;
        });
        float S;
        M = block_softmax_stats<NT>(m, s, red, &S);
        invS = 1.f / S;
        // red holds each wavefront's merged (max, sum): its range's share of
        // p0, the bonus weights while c = 0
        if (static_cast<int>(threadIdx.x) < (NT / kWave))
            wtot[threadIdx.x] = red[(NT / kWave) + threadIdx.x] * merge_scale(red[threadIdx.x], M) * invS;
    } else {
        float m = -INFINITY, s = 0.f;
        row_pass(a, lrow, nullptr, V, [&](int, float l, float) {
            const float mn = fmaxf(m, l);
            s = s * merge_scale(m, mn) + __expf(l - mn);
            m = mn;
        });
        float S;
        M = block_softmax_stats<NT>(m, s, red, &S);
        invS = 1.f / S;
    }
    if (threadIdx.x == 0) cd_sh[0] = make_float2(0.f, 1.f);
    float c = 0.f, D = 1.f;
    for (int i = 0; i < nk; ++i) {
        const float cn = c + D;
        float t = 0.f;
        if constexpr (RJ > 0) {
#pragma unroll
            for (int j = 0; j < RJ; ++j) t += fmaxf(pv[j] - cn * qv[j], 0.f);
        } else if constexpr (RJ < 0) {
            wave_pass(a, rr, true, vg0, vg1, [&](const float (&l)[8], const float (&q1)[8]) {
#pragma unroll
                for (int e = 0; e < 8; ++e) t += fmaxf(__expf(l[e] - M) * invS - cn * q1[e], 0.f);
            });
        } else {
            row_pass(a, lrow, qrow, V,
                     [&](int, float l, float q1) { t += fmaxf(__expf(l - M) * invS - cn * q1, 0.f); });
        }
        const float T = block_sum<NT>(t, red);
        if (T > 0.f) {
            c = cn;
            D = T;
            // red holds the wavefronts' sums of max(p0 - c q, 0) for the new c
            if (RJ < 0 && static_cast<int>(threadIdx.x) < (NT / kWave)) wtot[threadIdx.x] = red[threadIdx.x];
        }
        if (threadIdx.x == 0 && i + 1 < kMaxBeams) cd_sh[i + 1] = make_float2(c, D);
    }
    __syncthreads();
    if (kid >= 0) {
        const float2 cd = cd_sh[threadIdx.x];
        const float px = fmaxf(__expf(kl - M) * invS - cd.x * kq, 0.f) / cd.y;
        a.test[ubase + kid] = make_float2(px, kq);
    }
    const float ub = a.u_bonus[b];
    int bonus;
    if constexpr (RJ > 0)
        bonus = bonus_regs<RJ>(pv, qv, c, ub, red, redi, gsum);
    else if constexpr (RJ < 0)
        bonus = bonus_streamed_vec<NT>(a, rr, M, invS, c, ub, wtot, redi);
    else
        bonus = bonus_streamed(a, lrow, qrow, M, invS, c, ub, red, redi);
    if (threadIdx.x == 0) a.bonus[ubase + u] = min(bonus, V - 1);
}

// Register-resident rows of bf16 logits with V a multiple of 8, in
// persistent workgroups.  Each workgroup walks a contiguous range of the
// valid slots in (request, slot) order and, while it computes slot r, has
// slot r+1's loads in flight: its logits into registers (16-byte groups of
// 8 entries, as load_row_regs), its q into LDS by direct loads (chunk c of
// thread t at bytes (c*kRowT + t)*16, so every thread reads back its own
// entries without bank conflicts), and the logit and q of its children's
// tokens.  A row (192 KB at V = 32000) takes about as long to arrive at one
// CU's share of the HBM bandwidth as its statistics take to compute, so one
// workgroup per slot spent half its time waiting; here the two overlap.  A
// request's parent array is built once per workgroup, not once per slot.
// 512 threads of 64 entries each: the current row (p0 and q), the next
// row's logits and the statistics fit the 256 registers of two wavefronts
// per SIMD.  The statistics are those of k_stoch_node<32>, with these
// differences in how they are formed: block reductions over eight
// wavefronts instead of sixteen; p0 = 2^(l log2(e) - M log2(e)) (one
// multiply-add before the exponential); each residual pass keeps its
// per-group sums, which the bonus search reuses when that pass set c.
constexpr int kRowT = 512;               // threads per workgroup
constexpr int kRowNW = kRowT / kWave;    // wavefronts
constexpr int kRJ = 64;                  // entries per thread: rows of up to kRowT*kRJ
constexpr int kStreamT = 512;            // threads per workgroup of the streamed 16-byte path
struct RowsShared {
    // the small arrays first: their addresses then fit the 16-bit offset
    // field of LDS instructions instead of being held in registers
    float2 cd_sh[kMaxBeams];
    float red[2 * kRowNW];
    int redi[2 * kRowNW + 1];
    __attribute__((aligned(16))) float gsum[(kRJ / 8) * kRowNW];
    int kids[kMaxBeams];
    int nkids_sh;
    int loc_sh[2];
    int parent[kMaxSlots];
    int tok_sh[kMaxSlots];
    __attribute__((aligned(1024))) float qst[kRJ * kRowT];  // q of the next slot
};
__global__ __launch_bounds__(kRowT, 1) void k_stoch_rows(StochArgs a) {
    __shared__ RowsShared sm;
    float2 *const cd_sh = sm.cd_sh;
    float *const red = sm.red;
    int *const redi = sm.redi;
    float *const gsum = sm.gsum;
    int *const kids = sm.kids;
    int &nkids_sh = sm.nkids_sh;
    int *const loc_sh = sm.loc_sh;
    int *const parent = sm.parent;
    int *const tok_sh = sm.tok_sh;
    float *const qst = sm.qst;
    constexpr int NT = kRowT;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int B = a.B, W = a.W, L = a.L, V = a.V;
    const int P = W * L;
    auto plen_of = [&](int bb) { return min(max(a.plen[bb], 0), P); };

    // valid slots (u < packed_len[b]) numbered in (b, u) order; this
    // workgroup takes numbers [R*w/G, R*(w+1)/G)
    long long R = 0;
    for (int b0 = 0; b0 < B; b0 += NT) {
        const int bb = b0 + tid;
        int tot;
        block_scan_int<NT>(bb < B ? plen_of(bb) : 0, redi, tot);
        R += tot;
    }
    const long long r0 = R * blockIdx.x / gridDim.x, r1 = R * (blockIdx.x + 1) / gridDim.x;
    if (r0 >= r1) return;
    {
        long long carry = 0;
        for (int b0 = 0; b0 < B; b0 += NT) {
            const int bb = b0 + tid;
            const int n = bb < B ? plen_of(bb) : 0;
            int tot;
            const long long incl = carry + block_scan_int<NT>(n, redi, tot);
            if (bb < B && incl - n <= r0 && r0 < incl) {
                loc_sh[0] = bb;
                loc_sh[1] = static_cast<int>(r0 - (incl - n));
            }
            carry += tot;
        }
        __syncthreads();
    }
    int b = __builtin_amdgcn_readfirstlane(loc_sh[0]);
    int u = __builtin_amdgcn_readfirstlane(loc_sh[1]);
    int n = plen_of(b);

    // the request's tokens and parent array
    auto load_request = [&](int bb, int nn) {
        for (int i = tid; i < nn; i += NT) tok_sh[i] = a.ptok[static_cast<size_t>(bb) * P + i];
        build_parents<NT>(a, bb, nn, parent);  // its barriers also publish tok_sh
    };
    // slot (bb, uu)'s logits into registers, the logit (raw bf16 bits) and q
    // of child kidn's token, and its bonus uniform.  Every load here is consumed only at the
    // next slot's top: converting the logit now, or loading it only in the
    // threads with a child (a merge of old and new values), would make the
    // compiler wait for it -- and so for every load issued before it.
    auto issue = [&](int bb, int uu, int kidn, u32x4 (&lr)[kRJ / 8], uint32_t &klr_o, float &kq_o, float &ub_o) {
        const size_t lrow = (static_cast<size_t>(bb) * P + uu) * static_cast<size_t>(V);
        // the lane's byte offsets are formed here from one opaque base: hoisted
        // out of the loop, two dozen of them would be held in registers
        uint32_t t16 = static_cast<uint32_t>(tid) * 16u;
        asm volatile("" : "+v"(t16));
        const rsrc_t rl = make_rsrc(static_cast<const uint16_t *>(a.logits) + lrow, static_cast<uint32_t>(V) * 2u);
#pragma unroll
        for (int g = 0; g < kRJ / 8; ++g)
            lr[g] = __builtin_amdgcn_raw_buffer_load_b128(rl, t16 + static_cast<uint32_t>(NT * g) * 16u, 0, 0);
        const int x = min(max(tok_sh[max(kidn, 0)], 0), V - 1);
        klr_o = static_cast<const uint16_t *>(a.logits)[lrow + x];
        kq_o = a.q[lrow + x];
        ub_o = a.u_bonus[bb];
    };

    // quarter hh of slot (bb, uu)'s q, by direct loads into LDS.  The
    // quarters go out at four points of the current slot's statistics (with
    // the logits, after the max, after the sum, after the residual passes):
    // issued together with the rest (24 wide loads per thread) they held each
    // wavefront at the load issue long enough to delay those statistics
    // (dedup sweep p = 0.1: 1292 -> 1131 us; the last quarter before the
    // bonus search rather than after it: 1103 us).
    auto issue_q = [&](int bb, int uu, int hh) {
        const size_t lrow = (static_cast<size_t>(bb) * P + uu) * static_cast<size_t>(V);
        uint32_t t16 = static_cast<uint32_t>(tid) * 16u;
        asm volatile("" : "+v"(t16));
        const i32x4_t rq = make_srsrc(a.q + lrow, static_cast<uint32_t>(V) * 4u);
        const uint32_t qdst = lds_addr_of(qst) + wave * 1024;
#pragma unroll
        for (int g = hh * (kRJ / 32); g < (hh + 1) * (kRJ / 32); ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                lds_dma16(qdst + (2 * g + h) * NT * 16, rq, 2u * t16 + static_cast<uint32_t>(NT * g) * 32u + 16u * h);
    };
    load_request(b, n);
    int nk = children_of<NT>(u, n, parent, kids, redi, &nkids_sh);
    int kid = tid < nk ? kids[tid] : -1;
    u32x4 lr[kRJ / 8];
    uint32_t klr;
    float kq, ub;
    issue(b, u, kid, lr, klr, kq, ub);
    issue_q(b, u, 0);
    issue_q(b, u, 1);
    issue_q(b, u, 2);
    issue_q(b, u, 3);

    for (long long r = r0; r < r1; ++r) {
        // slot r's loads have landed (every thread's share, after the barrier)
        vm_wait<0>();
        __syncthreads();
        float pv[kRJ], qv[kRJ];  // logits, then p0, and q of this thread's entries x = reg_x<NT>(j)
        // V is a multiple of 8, so each 8-entry group lies wholly inside or
        // wholly past the row: the logits of groups past it are set to -inf
        // (p0 = 0 there, no masks below); q past the row reads as zero
#pragma unroll
        for (int g = 0; g < kRJ / 8; ++g) {
            // group g lies inside the row for every thread when 8*NT*(g+1) <= V
            // (a uniform test): only the groups reaching past V are masked
            const bool gin = 8 * NT * (g + 1) <= V || reg_x<NT>(8 * g) < V;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t wv = gin ? lr[g][k] : 0xFF80FF80u;
                pv[8 * g + 2 * k] = __uint_as_float(wv << 16);
                pv[8 * g + 2 * k + 1] = __uint_as_float(wv & 0xFFFF0000u);
            }
            const float4 q0 = *reinterpret_cast<const float4 *>(qst + ((2 * g) * NT + tid) * 4);
            const float4 q1 = *reinterpret_cast<const float4 *>(qst + ((2 * g + 1) * NT + tid) * 4);
            qv[8 * g + 0] = q0.x;
            qv[8 * g + 1] = q0.y;
            qv[8 * g + 2] = q0.z;
            qv[8 * g + 3] = q0.w;
            qv[8 * g + 4] = q1.x;
            qv[8 * g + 5] = q1.y;
            qv[8 * g + 6] = q1.z;
            qv[8 * g + 7] = q1.w;
        }
        // slot r's values, held while slot r+1's loads go out (the asm keeps
        // the compiler from waiting for them later, behind the new loads)
        const int cb = b, cu = u, cnk = nk, ckid = kid;
        float ckq = kq, cub = ub;
        uint32_t cklr = klr;
        asm volatile("" : "+v"(cklr), "+v"(ckq), "+v"(cub));
        const float ckl = __uint_as_float(cklr << 16);
        __syncthreads();  // every thread has read q from LDS
        if (r + 1 < r1) {
            if (++u >= n) {
                do {
                    ++b;
                    n = plen_of(b);
                } while (n == 0);
                u = 0;
                load_request(b, n);
            }
            nk = children_of<NT>(u, n, parent, kids, redi, &nkids_sh);
            kid = tid < nk ? kids[tid] : -1;
            issue(b, u, kid, lr, klr, kq, ub);
            issue_q(b, u, 0);
        }

        // slot r: softmax statistics from registers
        const size_t ubase = static_cast<size_t>(cb) * P;
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < kRJ; ++j) m = fmaxf(m, pv[j]);
        const float M = block_max<NT>(m, red);
        if (r + 1 < r1) issue_q(b, u, 1);
        // exp(l - M) as 2^(l log2(e) - M log2(e)): one multiply-add, no subtraction
        // (v_exp_f32 as __expf uses it: results below the normal range flush to 0)
        const float ML = M * kLog2e;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < kRJ; ++j) {
            pv[j] = fast_exp2(fmaf(pv[j], kLog2e, -ML));
            s += pv[j];
        }
        const float invS = 1.f / block_sum<NT>(s, red);
        if (r + 1 < r1) issue_q(b, u, 2);
#pragma unroll
        for (int j = 0; j < kRJ; ++j) pv[j] *= invS;
        if (tid == 0) cd_sh[0] = make_float2(0.f, 1.f);
        // each pass keeps its per-group sums: when the last pass sets c they
        // are the bonus weights' group sums already
        float c = 0.f, D = 1.f;
        float tsk[kRJ / 8];
        bool have = false;
        for (int i = 0; i < cnk; ++i) {
            const float cn = c + D;
            float t = 0.f;
#pragma unroll
            for (int g = 0; g < kRJ / 8; ++g) {
                float tg = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) tg += fmaxf(pv[8 * g + e] - cn * qv[8 * g + e], 0.f);
                tsk[g] = tg;
                t += tg;
            }
            const float T = block_sum<NT>(t, red);
            have = T > 0.f;
            if (have) {
                c = cn;
                D = T;
            }
            if (tid == 0 && i + 1 < kMaxBeams) cd_sh[i + 1] = make_float2(c, D);
        }
        __syncthreads();
        if (r + 1 < r1) issue_q(b, u, 3);
        if (ckid >= 0) {
            const float2 cd = cd_sh[tid];
            const float px = fmaxf(fast_exp2(fmaf(ckl, kLog2e, -ML)) * invS - cd.x * ckq, 0.f) / cd.y;
            a.test[ubase + ckid] = make_float2(px, ckq);
        }
        const int bonus = bonus_regs<kRJ, NT>(pv, qv, c, cub, red, redi, gsum, tsk, have);
        if (tid == 0) a.bonus[ubase + cu] = min(bonus, V - 1);
    }
    vm_wait<0>();
}

// The whole workgroup stages the request's test pairs, uniforms and parent
// array (one load per thread: a single wavefront needed eight dependent
// round trips at 512 slots); the walk itself is sequential, so wavefront 0
// alone does it: the children of a node are the slots above it whose parent
// it is, found in slot order 64 slots at a time by a ballot, and tested in
// that order -- no block-wide scans or barriers per depth.
constexpr int kWalkT = kT;
__global__ __launch_bounds__(kWalkT) void k_stoch_walk(StochArgs a) {
    __shared__ int parent[kMaxSlots];
    __shared__ float2 test_sh[kMaxSlots];  // (p_i(x), q(x)) of each slot's test at its parent
    __shared__ float ua_sh[kMaxBeamLen * kMaxBeams];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int W = a.W, L = a.L;
    const int P = W * L;
    const int n = min(max(a.plen[b], 0), P);
    int32_t *acc_row = a.accepted + static_cast<size_t>(b) * L;
    int32_t *path_row = a.path ? a.path + static_cast<size_t>(b) * L : nullptr;
    for (int i = lane; i < L; i += kWalkT) {
        acc_row[i] = -1;
        if (path_row) path_row[i] = -1;
    }
    if (n == 0) {
        if (lane == 0) {
            a.best_beam[b] = -1;
            a.accept_len[b] = -1;
        }
        return;
    }
    const int32_t *un = a.unpacker + static_cast<size_t>(b) * P;
    const size_t ubase = static_cast<size_t>(b) * P;
    for (int i = lane; i < n; i += kWalkT) test_sh[i] = a.test[ubase + i];
    for (int i = lane; i < L * W; i += kWalkT) ua_sh[i] = a.u_acc[static_cast<size_t>(b) * L * W + i];
    build_parents<kWalkT>(a, b, n, parent);  // its barriers also publish the staging above
    if (threadIdx.x >= kWave) return;         // no barrier follows: wavefront 0 walks
    int u = 0, d = 0;
    while (true) {
        // a node at depth L-1 is a leaf (bounds the walk on any unpacker)
        int next = -1;
        if (d + 1 < L) {
            int rank = 0;  // children of u tested so far (at most kMaxBeams, as their count is)
            for (int c0 = u + 1; c0 < n && next < 0 && rank < kMaxBeams; c0 += kWave) {
                const int cs = c0 + lane;
                uint64_t kidbits = __ballot(cs < n && parent[cs] == u);
                while (kidbits && next < 0 && rank < kMaxBeams) {  // the same values in every lane
                    const int ch = c0 + __ffsll(static_cast<long long>(kidbits)) - 1;
                    kidbits &= kidbits - 1;
                    const float r = ua_sh[d * W + min(rank, W - 1)];
                    const float2 t = test_sh[ch];
                    if (r * t.y < t.x) next = ch;
                    ++rank;
                }
            }
        }
        if (next < 0) break;
        if (lane == 0) {
            acc_row[d] = a.ptok[ubase + next];
            if (path_row) path_row[d + 1] = next;
        }
        u = next;
        ++d;
    }
    if (lane == 0) {
        if (path_row) path_row[0] = 0;
        acc_row[d] = a.bonus[ubase + u];
        a.accept_len[b] = d;
        int best = -1;
        for (int w = 0; w < W && best < 0; ++w)
            if (un[w * L + d] == u) best = w;
        a.best_beam[b] = best;
    }
}

}  // namespace

size_t stochastic_workspace_bytes(int B, int W, int L) {
    const size_t slots = static_cast<size_t>(B) * W * L;
    return slots * (sizeof(float2) + sizeof(int32_t));
}

hipError_t launch_stochastic_accept(int dtype, const int32_t *unpacker, const int32_t *plen, const int32_t *ptok,
                                    const void *logits, const float *q, const float *u_accept, const float *u_bonus,
                                    int B, int W, int L, int V, int32_t *best_beam, int32_t *accept_len,
                                    int32_t *accepted, int32_t *path, void *ws, hipStream_t stream) {
    StochArgs a{unpacker, plen, ptok, logits, q, u_accept, u_bonus, B, W, L, V, dtype == 1 ? 1 : 0,
                best_beam, accept_len, accepted, path, static_cast<float2 *>(ws),
                reinterpret_cast<int32_t *>(static_cast<float2 *>(ws) + static_cast<size_t>(B) * W * L)};
    const size_t slots = static_cast<size_t>(B) * W * L;
    const dim3 grid(static_cast<unsigned>(slots));
    if (dtype == 1 && V % 8 == 0 && V <= kRowT * kRJ) {
        // persistent: one workgroup per CU (fewer when there are fewer slots)
        const unsigned g = static_cast<unsigned>(std::min<size_t>(slots, static_cast<size_t>(device_cu_count())));
        hipLaunchKernelGGL(k_stoch_rows, dim3(g), dim3(kRowT), 0, stream, a);
    } else if (V <= kT * 32)
        hipLaunchKernelGGL(k_stoch_node<32>, grid, dim3(kT), 0, stream, a);
    else if (V % 8 == 0)
        // 512 threads, two workgroups per CU: one workgroup's reductions and
        // single-wavefront bonus scan overlap the other's streamed passes
        hipLaunchKernelGGL((k_stoch_node<-1, kStreamT>), grid, dim3(kStreamT), 0, stream, a);
    else
        hipLaunchKernelGGL(k_stoch_node<0>, grid, dim3(kT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_stoch_walk, dim3(B), dim3(kWalkT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rd
