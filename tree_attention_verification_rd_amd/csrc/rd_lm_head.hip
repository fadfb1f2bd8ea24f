// Step 3: output projection and greedy target token.
//
// Greedy verification (Apple/NVIDIA ReDrafter news article, greedy-decoding
// benchmark paragraph) needs the target's argmax over the vocabulary at
// every packed position: logits = hidden . W^T, argmax taken on the fp32
// accumulators with the lowest vocabulary id winning ties.
//
// bf16 GEMM layout.  Only valid packed rows (p < packed_len[b]) are
// computed: a small kernel compacts them into a row map.  The product is
// formed transposed, C^T = W X^T, so that
//   - the A operand is W: each wavefront streams its own vocabulary rows
//     from HBM straight into registers (no LDS round trip -- no other
//     wavefront needs them), kept NPF k-steps ahead in a register ring;
//   - the B operand is X (hidden rows), shared by every wavefront of the
//     workgroup and staged through double-buffered LDS;
//   - each lane's accumulator holds four consecutive vocabulary entries of
//     one row, which is what the argmax epilogue and the logits store want.
// Per workgroup: 4 wavefronts x VW vocabulary rows, BR compact rows, K in
// steps of 64.  The epilogue reduces (max, first index) over the tile's
// vocabulary range and writes one partial per (row, vocabulary tile); a
// second kernel reduces the partials in a fixed order.
#include <math.h>

#include "rd_common.h"
#include "rd_internal.h"

namespace rd {

namespace {

constexpr int kBK = 64;

struct LmArgs {
    const uint16_t *hidden, *weight;
    const int32_t *rowmap;
    const int32_t *rcount;
    int B, P, K, V;
    uint16_t *logits;
    float *pval;
    int32_t *pidx;
    int nvt, nrt;
};

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// valid rows -> compact row map (rowmap[m] = b*P + p), and their count
__global__ __launch_bounds__(256) void k_rowmap(const int32_t *__restrict__ plen, int B, int P,
                                                int32_t *__restrict__ rowmap, int32_t *__restrict__ rcount) {
    __shared__ int scan[256];
    __shared__ int carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int b0 = 0; b0 < B; b0 += 256) {
        const int b = b0 + threadIdx.x;
        const int n = (b < B) ? (plen ? min(max(plen[b], 0), P) : P) : 0;
        scan[threadIdx.x] = n;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int add = (threadIdx.x >= off) ? scan[threadIdx.x - off] : 0;
            __syncthreads();
            scan[threadIdx.x] += add;
            __syncthreads();
        }
        const int start = carry + scan[threadIdx.x] - n;
        for (int p = 0; p < n; ++p) rowmap[start + p] = b * P + p;
        __syncthreads();
        if (threadIdx.x == 255) carry += scan[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) *rcount = carry;
}

template <int VW, int BR, int NPF, int MINB>
__global__ __launch_bounds__(256, MINB) void k_lm_head_bf16(LmArgs a) {
    constexpr int NVB = VW / 16;
    constexpr int NRB = BR / 16;
    constexpr int XS = kBK + 8;          // LDS row stride (elements)
    constexpr int XLD = BR * (kBK / 8) / 256;  // 16-byte pieces per thread per k-step
    static_assert(NPF % 2 == 0, "the LDS buffer index must be static inside the unrolled ring");
    __shared__ uint16_t xs[2][BR * XS];
    __shared__ float redv[4][BR];
    __shared__ int32_t redi[4][BR];

    // wave-uniform values are read into scalar registers explicitly so the
    // buffer resources built from them stay scalar (no per-lane loops)
    const int R = __builtin_amdgcn_readfirstlane(*a.rcount);
    const int ntiles = a.nrt * a.nvt;
    const int t = xcd_tile(blockIdx.x, ntiles);
    // groups of up to 8 row tiles walk the vocabulary together
    constexpr int GM = 8;
    const int grp = t / (GM * a.nvt);
    const int gsz = min(GM, a.nrt - grp * GM);
    const int within = t - grp * GM * a.nvt;
    const int rt = grp * GM + within % gsz;
    const int vt = within / gsz;
    const int r0 = rt * BR;
    if (r0 >= R) return;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 15;
    const int kg = lane >> 4;
    const int vw0 = vt * 4 * VW + wave * VW;
    const int rvalid = min(BR, R - r0);
    const int nrb = (rvalid + 15) / 16;
    const int K = a.K;
    const int nk = (K + kBK - 1) / kBK;

    // Buffer loads: one resource over this wavefront's W rows (rows past V
    // fall outside it) and one over all hidden rows.  Out-of-range rows and
    // k-chunks get an out-of-range offset and read as zeros, so every
    // thread issues the same loads on every path.
    const int nk_pad = (nk + NPF - 1) / NPF * NPF;
    const uint32_t rowb = static_cast<uint32_t>(K) * 2;
    const int wrows = max(0, min(a.V, vw0 + VW) - vw0);
    const i32x4_t wres = make_srsrc(a.weight + static_cast<size_t>(min(vw0, a.V)) * K,
                                    static_cast<uint32_t>(wrows) * rowb);
    const i32x4_t xres = make_srsrc(a.hidden, static_cast<uint32_t>(static_cast<size_t>(a.B) * a.P * K * 2));
    uint32_t woff[NVB];
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) woff[vb] = (vb * 16 + lq) * rowb + 16 * kg;
    uint32_t xoff[XLD];
#pragma unroll
    for (int j = 0; j < XLD; ++j) {
        const int c = tid + 256 * j;
        const int m = r0 + c / 8;
        xoff[j] = (m < R) ? static_cast<uint32_t>(a.rowmap[m]) * rowb + 16 * (c % 8) : kOOB;
    }

    // Each vocabulary tile walks K from its own starting k-step (wrapping),
    // so that concurrent tiles do not all address the same offset within
    // their power-of-two-strided rows (which would crowd a few HBM
    // channels).  The start depends on the vocabulary tile only: the row
    // tiles that share these weight rows run side by side on one XCD and
    // must walk K in the same order to share each chunk through L2.
    // Stages are loaded in k order, so the rotated index is advanced
    // incrementally; padding k-steps (kt >= nk) read zeros.
    const int krot = (vt * 5) % nk;
    int kload = 0;          // next k-step to load (unrotated)
    int kload_rot = krot;   // its rotated index
    auto next_kstep = [&]() {
        const int kr = kload < nk ? kload_rot : nk;
        ++kload;
        kload_rot = (kload_rot + 1 == nk) ? 0 : kload_rot + 1;
        return kr;
    };
    auto load_stage = [&](u32x4 (&w)[NVB][2], u32x4 (&x)[XLD]) {
        const int kr = next_kstep();
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bool in = kr * kBK + 32 * ks + 8 * kg < K;
                ring_load16(w[vb][ks], wres, in ? woff[vb] + (kr * kBK + 32 * ks) * 2 : kOOB);
            }
#pragma unroll
        for (int j = 0; j < XLD; ++j) {
            const int c = tid + 256 * j;
            const bool in = xoff[j] != kOOB && kr * kBK + 8 * (c % 8) < K;
            ring_load16(x[j], xres, in ? xoff[j] + kr * kBK * 2 : kOOB);
        }
    };
    constexpr int kStageLoads = NVB * 2 + XLD;
    // wait until stage `st` has landed: the NPF-1 younger stages stay in flight
    auto stage_ready = [&](u32x4 (&w)[NVB][2], u32x4 (&x)[XLD]) {
        vm_wait<(NPF - 1) * kStageLoads>();
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) asm volatile("" : "+v"(w[vb][ks]));
#pragma unroll
        for (int j = 0; j < XLD; ++j) asm volatile("" : "+v"(x[j]));
    };
    auto store_x = [&](const u32x4 (&src)[XLD], int buf) {
#pragma unroll
        for (int j = 0; j < XLD; ++j) {
            const int c = tid + 256 * j;
            *reinterpret_cast<u32x4 *>(&xs[buf][(c / 8) * XS + 8 * (c % 8)]) = src[j];
        }
    };

    f32x4 acc[NVB][NRB];
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) acc[vb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Stage ring: the W and X loads of k-step j are issued together, NPF
    // k-steps before j is computed, into register slot j % NPF.  Loads
    // complete in issue order, so the wait at k-step j only covers stage j
    // and the NPF-1 younger stages stay in flight.  X moves to LDS (double
    // buffered) right before its k-step; one barrier per k-step suffices.
    u32x4 wreg[NPF][NVB][2];
    u32x4 xreg[NPF][XLD];
#pragma unroll
    for (int st = 0; st < NPF; ++st) load_stage(wreg[st], xreg[st]);

    for (int kt0 = 0; kt0 < nk_pad; kt0 += NPF) {
#pragma unroll
        for (int st = 0; st < NPF; ++st) {
            const int kt = kt0 + st;
            const int buf = st & 1;  // == kt & 1 since NPF is even
            stage_ready(wreg[st], xreg[st]);
            store_x(xreg[st], buf);
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                // all X fragments of this half-step are read before the
                // MFMAs that use them, so LDS latency overlaps the MFMAs
                bf16x8 xb[NRB];
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb)
                    xb[rb] = as_bf16x8(ld16(&xs[buf][(rb * 16 + lq) * XS + 32 * ks + 8 * kg]));
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb)  // blocks past the valid rows multiply zeros
#pragma unroll
                    for (int vb = 0; vb < NVB; ++vb)
                        acc[vb][rb] = mfma16x16x32(as_bf16(wreg[st][vb][ks]), xb[rb], acc[vb][rb]);
            }
            load_stage(wreg[st], xreg[st]);
        }
    }

    // The ring's trailing prefetches (past K) are still landing: wait for
    // them with every slot tied, so that no register of an in-flight load
    // is handed to other code before the data has arrived.
    vm_wait<0>();
#pragma unroll
    for (int st = 0; st < NPF; ++st) {
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) asm volatile("" : "+v"(wreg[st][vb][ks]));
#pragma unroll
        for (int j = 0; j < XLD; ++j) asm volatile("" : "+v"(xreg[st][j]));
    }

    // epilogue: acc[vb][rb][e] = logit(row r0 + rb*16 + lq, vocab vw0 + vb*16 + 4*kg + e)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        if (rb < nrb) {
            const int m = r0 + rb * 16 + lq;
            const bool mvalid = m < R;
            const int pr = mvalid ? a.rowmap[m] : 0;
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                const int v = vw0 + vb * 16 + 4 * kg;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (v + e < a.V && better(acc[vb][rb][e], v + e, bv, bi)) {
                        bv = acc[vb][rb][e];
                        bi = v + e;
                    }
                if (a.logits && mvalid) {
                    uint16_t *dst = a.logits + static_cast<size_t>(pr) * a.V + v;
                    if (v + 3 < a.V && (a.V % 4 == 0)) {
                        u16x4 w = {f32_to_bf16_bits(acc[vb][rb][0]), f32_to_bf16_bits(acc[vb][rb][1]),
                                   f32_to_bf16_bits(acc[vb][rb][2]), f32_to_bf16_bits(acc[vb][rb][3])};
                        *reinterpret_cast<u16x4 *>(dst) = w;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (v + e < a.V) dst[e] = f32_to_bf16_bits(acc[vb][rb][e]);
                    }
                }
            }
        }
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            const float ov = shfl_xor(bv, off);
            const int oi = shfl_xor(bi, off);
            if (better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (kg == 0) {
            redv[wave][rb * 16 + lq] = bv;
            redi[wave][rb * 16 + lq] = bi;
        }
    }
    __syncthreads();
    for (int i = tid; i < rvalid; i += 256) {
        float bv = redv[0][i];
        int bi = redi[0][i];
#pragma unroll
        for (int w = 1; w < 4; ++w)
            if (better(redv[w][i], redi[w][i], bv, bi)) {
                bv = redv[w][i];
                bi = redi[w][i];
            }
        const size_t pr = static_cast<size_t>(a.rowmap[r0 + i]);
        a.pval[pr * a.nvt + vt] = bv;
        a.pidx[pr * a.nvt + vt] = bi;
    }
}

// fp32 path: one workgroup per (padded row, 256-wide vocabulary tile)
__global__ __launch_bounds__(256) void k_lm_head_f32(const float *__restrict__ hidden,
                                                     const int32_t *__restrict__ plen,
                                                     const float *__restrict__ weight, int P, int K, int V,
                                                     float *__restrict__ logits, float *__restrict__ pval,
                                                     int32_t *__restrict__ pidx, int nvt) {
    __shared__ float hs[1024];
    __shared__ float rv[256];
    __shared__ int32_t ri[256];
    const int vt = blockIdx.x % nvt;
    const size_t pr = blockIdx.x / nvt;
    const int b = static_cast<int>(pr / P);
    const int p = static_cast<int>(pr % P);
    const int Pb = plen ? min(max(plen[b], 0), P) : P;
    if (p >= Pb) return;
    const int v = vt * 256 + threadIdx.x;
    const float *wr = weight + static_cast<size_t>(min(v, V - 1)) * K;
    float acc = 0.f;
    for (int k0 = 0; k0 < K; k0 += 1024) {
        const int kn = min(1024, K - k0);
        __syncthreads();
        for (int k = threadIdx.x; k < kn; k += 256) hs[k] = hidden[pr * K + k0 + k];
        __syncthreads();
        for (int k = 0; k < kn; ++k) acc = fmaf(hs[k], wr[k0 + k], acc);
    }
    if (v < V && logits) logits[pr * V + v] = acc;
    rv[threadIdx.x] = (v < V) ? acc : -INFINITY;
    ri[threadIdx.x] = (v < V) ? v : 0x7fffffff;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off &&
            better(rv[threadIdx.x + off], ri[threadIdx.x + off], rv[threadIdx.x], ri[threadIdx.x])) {
            rv[threadIdx.x] = rv[threadIdx.x + off];
            ri[threadIdx.x] = ri[threadIdx.x + off];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        pval[pr * nvt + vt] = rv[0];
        pidx[pr * nvt + vt] = ri[0];
    }
}

// final argmax per padded row: one wavefront per row, partials in a fixed order
__global__ __launch_bounds__(256) void k_argmax_reduce(const float *__restrict__ pval,
                                                       const int32_t *__restrict__ pidx,
                                                       const int32_t *__restrict__ plen, int B, int P, int nvt,
                                                       int32_t *__restrict__ argmax) {
    const size_t pr = static_cast<size_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (pr >= static_cast<size_t>(B) * P) return;
    const int b = static_cast<int>(pr / P);
    const int p = static_cast<int>(pr % P);
    const int Pb = plen ? min(max(plen[b], 0), P) : P;
    if (p >= Pb) {
        if (lane == 0) argmax[pr] = -1;
        return;
    }
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = lane; i < nvt; i += kWave) {
        const float v = pval[pr * nvt + i];
        const int ix = pidx[pr * nvt + i];
        if (better(v, ix, bv, bi)) {
            bv = v;
            bi = ix;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = shfl_xor(bv, off);
        const int oi = shfl_xor(bi, off);
        if (better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    if (lane == 0) argmax[pr] = bi;
}

constexpr size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

constexpr int kVocabPerWave = 32;
constexpr int kRowTile = 128;

}  // namespace

LmPlan plan_lm_head(int dtype, int B, int P_max, int K, int V) {
    LmPlan plan{};
    plan.rows_pad = B * P_max;
    if (dtype == 0) {
        plan.vtile = 256;
    } else {
        plan.vtile = 4 * kVocabPerWave;
    }
    plan.nvt = (V + plan.vtile - 1) / plan.vtile;
    const size_t rows = static_cast<size_t>(plan.rows_pad);
    plan.ws_bytes = 256 + align256(rows * 4) + 2 * align256(rows * plan.nvt * 4);
    return plan;
}

hipError_t launch_lm_head(int dtype, const LmPlan &plan, const void *hidden, const int32_t *plen,
                          const void *weight, int B, int P_max, int K, int V, void *logits, int32_t *argmax,
                          void *ws, hipStream_t stream) {
    char *w = static_cast<char *>(ws);
    int32_t *rcount = reinterpret_cast<int32_t *>(w);
    int32_t *rowmap = reinterpret_cast<int32_t *>(w + 256);
    const size_t rows = static_cast<size_t>(plan.rows_pad);
    float *pval = reinterpret_cast<float *>(w + 256 + align256(rows * 4));
    int32_t *pidx = reinterpret_cast<int32_t *>(w + 256 + align256(rows * 4) + align256(rows * plan.nvt * 4));

    if (dtype == 0) {
        hipLaunchKernelGGL(k_lm_head_f32, dim3(static_cast<unsigned>(rows * plan.nvt)), dim3(256), 0, stream,
                           static_cast<const float *>(hidden), plen, static_cast<const float *>(weight), P_max, K,
                           V, static_cast<float *>(logits), pval, pidx, plan.nvt);
    } else {
        hipLaunchKernelGGL(k_rowmap, dim3(1), dim3(256), 0, stream, plen, B, P_max, rowmap, rcount);
        LmArgs a;
        a.hidden = static_cast<const uint16_t *>(hidden);
        a.weight = static_cast<const uint16_t *>(weight);
        a.rowmap = rowmap;
        a.rcount = rcount;
        a.B = B;
        a.P = P_max;
        a.K = K;
        a.V = V;
        a.logits = static_cast<uint16_t *>(logits);
        a.pval = pval;
        a.pidx = pidx;
        a.nvt = plan.nvt;
        // 4 wavefronts x 32 vocabulary rows, 128 compact rows per workgroup,
        // two-stage load ring, two workgroups per CU: the best of the tile
        // shapes measured on MI355X for both the few-row and many-row cases
        a.nrt = static_cast<int>((rows + kRowTile - 1) / kRowTile);
        hipLaunchKernelGGL((k_lm_head_bf16<kVocabPerWave, kRowTile, 2, 2>), dim3(static_cast<unsigned>(a.nrt * a.nvt)),
                           dim3(256), 0, stream, a);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_argmax_reduce, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, stream, pval,
                       pidx, plen, B, P_max, plan.nvt, argmax);
    return hipGetLastError();
}

}  // namespace rd
