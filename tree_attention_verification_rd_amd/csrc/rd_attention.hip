// Step 2: tree attention over the packed tokens.
//
// ReDrafter verifies every candidate path of the beam tree in one pass
// (TensorRT-LLM ReDrafter blog, intro and FAQ; Apple/NVIDIA news article,
// "Dynamic tree attention").  Packed query p attends to all cached keys of
// its request and to the packed keys whose bit is set in its tree-mask row
// (SpecInfer's topology-aware causal mask, speculative-decoding survey,
// "Token Tree Verifier").
//
// bf16 kernel layout.  One workgroup (4 wavefronts) handles 64 query rows of
// one (request, KV head) and one split of the KV cache; row r of the
// (request, KV head) is packed token r / G, query head g*G + r % G, so the G
// heads sharing a KV head share every K/V tile.  Keys stream through LDS in
// tiles of 64: cache tiles first, then (last split only) the packed tiles up
// to the largest token of the block -- parents precede children, so later
// tokens cannot be ancestors.
//
// Each wavefront owns 16 query rows.  Scores are computed transposed,
// S^T = K Q^T (A = K rows from LDS, B = Q held in registers), so each lane's
// accumulator column is one query and the probabilities P^T come out of the
// MFMA already in the B-operand layout of O^T = V^T P^T; only V is
// transposed, once, when a tile is written to LDS.  Online softmax runs in
// fp32 in the log2 domain.  With more than one split, each split writes
// (max, sum, unnormalised O) in fp32 and a combine kernel merges them.
#include <math.h>
#include <stdlib.h>

#include "rd_common.h"
#include "rd_internal.h"

namespace rd {

namespace {

constexpr int kBlockM = 64;  // query rows per workgroup
constexpr int kBlockN = 64;  // keys per tile
constexpr int kMaxSplits = 64;
constexpr int kMaxMaskWords = (kMaxBeams * kMaxBeamLen) / 32;

struct AttnArgs {
    const uint16_t *q, *k_new, *v_new, *k_cache, *v_cache;
    const int32_t *kv_len;
    const uint32_t *mask;
    const int32_t *plen;
    int B, P, Hq, Hkv, G, S_max, nw;
    float scale_log2;
    int nqblk, nsplit, chunk;
    uint16_t *out;
    float *ws_o;    // [B, Hkv, nsplit, nqblk*64, D]
    float2 *ws_ml;  // [B, Hkv, nsplit, nqblk*64]
};

template <int D>
struct AttnSmem {
    static constexpr int KS = D + 8;        // K row stride (elements)
    static constexpr int VS = kBlockN + 8;  // V^T row stride (elements)
    uint16_t k[kBlockN * KS];
    uint16_t vt[D * VS];
};

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

template <int D>
__global__ __launch_bounds__(256) void k_tree_attn_bf16(AttnArgs a) {
    constexpr int NKC = D / 32;          // k-steps over the head dim (QK^T)
    constexpr int NDB = D / 16;          // 16-row blocks of the head dim (PV)
    constexpr int KCH = D / 8;           // 16-byte chunks per key row
    constexpr int KLD = kBlockN * KCH / 256;  // K chunks per thread per tile
    using Smem = AttnSmem<D>;
    __shared__ Smem smem[2];
    __shared__ uint32_t mwords[kBlockM * kMaxMaskWords];  // tree-mask rows of this block's tokens

    const int ntiles = a.B * a.Hkv * a.nsplit * a.nqblk;
    const int t = xcd_tile(blockIdx.x, ntiles);
    const int qb = t % a.nqblk;
    int rest = t / a.nqblk;
    const int s = rest % a.nsplit;
    rest /= a.nsplit;
    const int g = rest % a.Hkv;
    const int b = rest / a.Hkv;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lq = lane & 15;
    const int kg = lane >> 4;

    const int Pb = min(max(a.plen[b], 0), a.P);
    const int kvl = min(max(a.kv_len[b], 0), a.S_max);
    const int Mb = a.G * Pb;
    const int Mpad = a.G * a.P;
    const int row0 = qb * kBlockM;

    if (row0 >= Mb) {
        // no valid query rows: with a single split this block owns the
        // padding rows of the output and writes them as zeros
        if (a.nsplit == 1) {
            for (int i = tid; i < kBlockM * KCH; i += 256) {
                const int r = row0 + i / KCH;
                if (r >= Mpad) continue;
                const int pz = r / a.G, hz = g * a.G + r % a.G;
                *reinterpret_cast<uint4 *>(a.out + ((static_cast<size_t>(b) * a.P + pz) * a.Hq + hz) * D +
                                           (i % KCH) * 8) = make_uint4(0, 0, 0, 0);
            }
        }
        return;
    }

    const int c0 = s * a.chunk;
    const int c1 = min(c0 + a.chunk, kvl);
    const int ncache = (c1 > c0) ? (c1 - c0 + kBlockN - 1) / kBlockN : 0;
    int tok_hi = 0, npk = 0;
    if (s == a.nsplit - 1) {
        tok_hi = (min(row0 + kBlockM, Mb) - 1) / a.G + 1;
        npk = (tok_hi + kBlockN - 1) / kBlockN;
    }
    const int ntile = ncache + npk;

    // this lane's query row
    const int r = row0 + wave * 16 + lq;
    const bool rvalid = r < Mb;
    const int p = rvalid ? r / a.G : 0;
    const int h = g * a.G + (rvalid ? r % a.G : 0);
    bf16x8 qf[NKC];
    {
        const uint16_t *qrow = a.q + ((static_cast<size_t>(b) * a.P + p) * a.Hq + h) * D;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
            qf[kc] = as_bf16x8(rvalid ? ld16(qrow + 32 * kc + 8 * kg) : make_uint4(0, 0, 0, 0));
    }
    // tokens of this block and their tree-mask rows, staged in LDS once
    const int tok_lo = row0 / a.G;
    if (npk > 0) {
        const int ntok = tok_hi - tok_lo;
        const uint32_t *msrc = a.mask + (static_cast<size_t>(b) * a.P + tok_lo) * a.nw;
        for (int i = tid; i < ntok * a.nw; i += 256) mwords[i] = msrc[i];
    }
    const int lt = rvalid ? p - tok_lo : 0;

    // K/V rows of tile i: cache tiles come first, then the packed tiles.
    // Buffer loads with one resource per source: keys past the valid range
    // get an out-of-range offset and read as zeros, so every thread issues
    // the same loads on every path and no select is needed.
    const size_t cache_base = (static_cast<size_t>(b) * a.Hkv + g) * a.S_max * D;
    const size_t fresh_base = (static_cast<size_t>(b) * a.P * a.Hkv + g) * D;
    const uint32_t cache_bytes = static_cast<uint32_t>(min<size_t>(static_cast<size_t>(a.S_max) * D * 2, kMaxRange));
    const uint32_t fresh_bytes = static_cast<uint32_t>(min<size_t>(static_cast<size_t>(a.P) * a.Hkv * D * 2, kMaxRange));
    const rsrc_t rk_c = make_rsrc(a.k_cache + cache_base, cache_bytes);
    const rsrc_t rv_c = make_rsrc(a.v_cache + cache_base, cache_bytes);
    const rsrc_t rk_n = make_rsrc(a.k_new + fresh_base, fresh_bytes);
    const rsrc_t rv_n = make_rsrc(a.v_new + fresh_base, fresh_bytes);

    // V loader threads: 16 key quads x KCH head-dim chunks (all 256 threads
    // for D = 128); the others repeat a load and skip the store
    const bool vthread = tid < 16 * KCH;
    const int vkq = tid & 15;                   // key quad: keys 4*vkq .. 4*vkq+3
    const int vdc = vthread ? (tid >> 4) : 0;   // head-dim chunk: d = 8*vdc .. 8*vdc+7

    // Cache tiles are visited from a per-block starting tile (wrapping) so
    // that concurrent blocks, whose slabs sit at power-of-two strides, do
    // not all address the same offsets and crowd a few HBM channels.
    const int trot = ncache > 0 ? (b * 7 + g * 3 + qb * 5) % ncache : 0;
    auto load_tile = [&](uint4 (&kr)[KLD], uint4 (&vr)[4], int i) {
        const bool cache = i < ncache;
        const rsrc_t rk = cache ? rk_c : rk_n;
        const rsrc_t rv = cache ? rv_c : rv_n;
        const int ic = cache ? (i + trot) % ncache : 0;
        const int kbase = cache ? c0 + ic * kBlockN : (i - ncache) * kBlockN;
        const int klim = cache ? c1 : tok_hi;
        const uint32_t rowb = cache ? D * 2 : static_cast<uint32_t>(a.Hkv) * D * 2;
#pragma unroll
        for (int j = 0; j < KLD; ++j) {
            const int c = tid + 256 * j;
            const int key = kbase + c / KCH;
            kr[j] = buf_load16(rk, key < klim ? key * rowb + (c % KCH) * 16 : kOOB);
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int key = kbase + 4 * vkq + r4;
            vr[r4] = buf_load16(rv, key < klim ? key * rowb + vdc * 16 : kOOB);
        }
    };
    auto store_tile = [&](const uint4 (&kr)[KLD], const uint4 (&vr)[4], Smem &sm) {
#pragma unroll
        for (int j = 0; j < KLD; ++j) {
            const int c = tid + 256 * j;
            *reinterpret_cast<uint4 *>(&sm.k[(c / KCH) * Smem::KS + 8 * (c % KCH)]) = kr[j];
        }
        if (vthread) {
            u16x8 v[4];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) __builtin_memcpy(&v[r4], &vr[r4], 16);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                u16x4 col = {v[0][jj], v[1][jj], v[2][jj], v[3][jj]};
                *reinterpret_cast<u16x4 *>(&sm.vt[(8 * vdc + jj) * Smem::VS + 4 * vkq]) = col;
            }
        }
    };

    f32x4 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrun = kNegBig;
    float lpart = 0.f;

    auto compute_tile = [&](int i, const Smem &sm) {
        // S^T for 64 keys x this wave's 16 queries.  Per head-dim step the
        // four key blocks' fragments are read together and feed four
        // independent accumulators, so LDS latency overlaps the MFMAs.
        f32x4 sc[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            bf16x8 ka[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                ka[kb] = as_bf16x8(ld16(&sm.k[(kb * 16 + lq) * Smem::KS + 32 * kc + 8 * kg]));
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sc[kb] = mfma16x16x32(ka[kb], qf[kc], sc[kb]);
        }

        // scale and mask; key of sc[kb][e] within the tile is kb*16 + 4*kg + e
        if (i < ncache) {
            const int lim = c1 - (c0 + ((i + trot) % ncache) * kBlockN);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = kb * 16 + 4 * kg + e;
                    sc[kb][e] = (j < lim) ? sc[kb][e] * a.scale_log2 : -INFINITY;
                }
        } else {
            const int pt = i - ncache;
            const int wi = 2 * pt;
            const uint32_t w0 = mwords[lt * a.nw + wi];
            const uint32_t w1 = (wi + 1 < a.nw) ? mwords[lt * a.nw + wi + 1] : 0u;
            const int lim = tok_hi - pt * kBlockN;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = kb * 16 + 4 * kg + e;
                    const uint32_t wd = (j < 32) ? w0 : w1;
                    const bool vis = (j < lim) && ((wd >> (j & 31)) & 1u);
                    sc[kb][e] = vis ? sc[kb][e] * a.scale_log2 : -INFINITY;
                }
        }

        // online softmax (per query column; the four k-groups hold disjoint keys)
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, sc[kb][e]);
        tmax = fmaxf(tmax, shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, shfl_xor(tmax, 32));
        const float mnew = fmaxf(mrun, tmax);
        const float alpha = fast_exp2(mrun - mnew);
        mrun = mnew;
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sc[kb][e] = fast_exp2(sc[kb][e] - mnew);
                psum += sc[kb][e];
            }
        lpart = lpart * alpha + psum;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;

        // O^T += V^T P^T, two k-steps of 32 keys: slots 0-3 hold keys
        // 32*ks + 4*kg + (0..3), slots 4-7 keys 32*ks + 16 + 4*kg + (0..3)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pb[e] = static_cast<__bf16>(sc[2 * ks][e]);
                pb[4 + e] = static_cast<__bf16>(sc[2 * ks + 1][e]);
            }
            uint4 vv[NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const uint16_t *vrow = &sm.vt[(db * 16 + lq) * Smem::VS + 32 * ks + 4 * kg];
                const uint2 lo = *reinterpret_cast<const uint2 *>(vrow);
                const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 16);
                vv[db] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] = mfma16x16x32(as_bf16x8(vv[db]), pb, o[db]);
        }
    };

    // Two-stage ring: tile j's K/V loads are issued two tiles ahead into
    // register slot j % 2 and written to LDS buffer j % 2 just before use;
    // loads complete in issue order, so each wait covers only the oldest
    // stage.  One barrier per tile: buffer j % 2 is rewritten only after
    // every wave has passed the barrier of tile j + 1.
    uint4 kreg[2][KLD];
    uint4 vreg[2][4];
    const int ntile_pad = (ntile + 1) & ~1;
    load_tile(kreg[0], vreg[0], 0);
    load_tile(kreg[1], vreg[1], 1);
    for (int i0 = 0; i0 < ntile_pad; i0 += 2) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int i = i0 + st;
            store_tile(kreg[st], vreg[st], smem[st]);
            __syncthreads();
            if (i < ntile) compute_tile(i, smem[st]);
            load_tile(kreg[st], vreg[st], i + 2);
        }
    }

    float lsum = lpart + shfl_xor(lpart, 16);
    lsum += shfl_xor(lsum, 32);

    if (a.nsplit == 1) {
        // o[db][e] = O[query r][d = db*16 + 4*kg + e]
        if (r < Mpad) {
            const float inv = (rvalid && lsum > 0.f) ? 1.f / lsum : 0.f;
            const int pz = r / a.G, hz = g * a.G + r % a.G;
            uint16_t *orow = a.out + ((static_cast<size_t>(b) * a.P + pz) * a.Hq + hz) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                u16x4 w = {f32_to_bf16_bits(o[db][0] * inv), f32_to_bf16_bits(o[db][1] * inv),
                           f32_to_bf16_bits(o[db][2] * inv), f32_to_bf16_bits(o[db][3] * inv)};
                *reinterpret_cast<u16x4 *>(orow + db * 16 + 4 * kg) = w;
            }
        }
    } else if (rvalid) {
        const size_t prow = ((static_cast<size_t>(b) * a.Hkv + g) * a.nsplit + s) * (a.nqblk * kBlockM) + r;
        float *orow = a.ws_o + prow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4 *>(orow + db * 16 + 4 * kg) = o[db];
        if (kg == 0) a.ws_ml[prow] = make_float2(mrun, lsum);
    }
}

// Merge of the per-split partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
    constexpr int KCH4 = D / 4;  // float4 chunks per row
    __shared__ float wgt[kBlockM][kMaxSplits + 1];
    const int qb = blockIdx.x % a.nqblk;
    const int bg = blockIdx.x / a.nqblk;
    const int g = bg % a.Hkv;
    const int b = bg / a.Hkv;
    const int Pb = min(max(a.plen[b], 0), a.P);
    const int Mb = a.G * Pb;
    const int Mpad = a.G * a.P;
    const int row0 = qb * kBlockM;
    const size_t split_stride = static_cast<size_t>(a.nqblk) * kBlockM;
    const size_t base = (static_cast<size_t>(b) * a.Hkv + g) * a.nsplit * split_stride;

    if (threadIdx.x < kBlockM) {
        const int r = row0 + threadIdx.x;
        if (r < Mb) {
            float M = kNegBig;
            for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.ws_ml[base + s * split_stride + r].x);
            float den = 0.f;
            for (int s = 0; s < a.nsplit; ++s) {
                const float2 ml = a.ws_ml[base + s * split_stride + r];
                const float w = fast_exp2(ml.x - M);
                wgt[threadIdx.x][s] = w;
                den += w * ml.y;
            }
            const float inv = den > 0.f ? 1.f / den : 0.f;
            for (int s = 0; s < a.nsplit; ++s) wgt[threadIdx.x][s] *= inv;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kBlockM * KCH4; i += 256) {
        const int rl = i / KCH4;
        const int c = i % KCH4;
        const int r = row0 + rl;
        if (r >= Mpad) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (r < Mb) {
            for (int s = 0; s < a.nsplit; ++s) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(a.ws_o + (base + s * split_stride + r) * D + 4 * c);
                acc += wgt[rl][s] * v;
            }
        }
        const int pz = r / a.G, hz = g * a.G + r % a.G;
        u16x4 w = {f32_to_bf16_bits(acc[0]), f32_to_bf16_bits(acc[1]), f32_to_bf16_bits(acc[2]),
                   f32_to_bf16_bits(acc[3])};
        *reinterpret_cast<u16x4 *>(a.out + ((static_cast<size_t>(b) * a.P + pz) * a.Hq + hz) * D + 4 * c) = w;
    }
}

// fp32 path: one wavefront per (request, packed token, head); every lane
// runs an online softmax over a strided subset of the visible keys, then
// the 64 partial states are merged through LDS.
template <int D>
__global__ __launch_bounds__(64) void k_tree_attn_f32(const float *__restrict__ q, const float *__restrict__ k_new,
                                                      const float *__restrict__ v_new,
                                                      const float *__restrict__ k_cache,
                                                      const float *__restrict__ v_cache,
                                                      const int32_t *__restrict__ kv_len,
                                                      const uint32_t *__restrict__ mask,
                                                      const int32_t *__restrict__ plen, int P, int Hq,
                                                      int Hkv, int S_max, int nw, float scale_log2,
                                                      float *__restrict__ out) {
    __shared__ float qs[D];
    __shared__ float part[kWave][D + 1];
    __shared__ float ml[kWave][2];
    const int lane = threadIdx.x;
    const int h = blockIdx.x % Hq;
    const int p = (blockIdx.x / Hq) % P;
    const int b = blockIdx.x / (Hq * P);
    const int G = Hq / Hkv;
    const int g = h / G;
    const int Pb = min(max(plen[b], 0), P);
    const int kvl = min(max(kv_len[b], 0), S_max);
    float *orow = out + ((static_cast<size_t>(b) * P + p) * Hq + h) * D;
    if (p >= Pb) {
        for (int d = lane; d < D; d += kWave) orow[d] = 0.f;
        return;
    }
    const float *qrow = q + ((static_cast<size_t>(b) * P + p) * Hq + h) * D;
    for (int d = lane; d < D; d += kWave) qs[d] = qrow[d];
    __syncthreads();
    const uint32_t *mrow = mask + (static_cast<size_t>(b) * P + p) * nw;

    float m = kNegBig, l = 0.f;
    float o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = 0.f;
    for (int j = lane; j < kvl + Pb; j += kWave) {
        const float *kr, *vr;
        if (j < kvl) {
            kr = k_cache + ((static_cast<size_t>(b) * Hkv + g) * S_max + j) * D;
            vr = v_cache + ((static_cast<size_t>(b) * Hkv + g) * S_max + j) * D;
        } else {
            const int pk = j - kvl;
            if (!((mrow[pk >> 5] >> (pk & 31)) & 1u)) continue;
            kr = k_new + ((static_cast<size_t>(b) * P + pk) * Hkv + g) * D;
            vr = v_new + ((static_cast<size_t>(b) * P + pk) * Hkv + g) * D;
        }
        float sdot = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) sdot = fmaf(qs[d], kr[d], sdot);
        const float s2 = sdot * scale_log2;
        const float mn = fmaxf(m, s2);
        const float alpha = fast_exp2(m - mn);
        const float pe = fast_exp2(s2 - mn);
        l = l * alpha + pe;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(pe, vr[d], o[d] * alpha);
        m = mn;
    }
    ml[lane][0] = m;
    ml[lane][1] = l;
    __syncthreads();
    float M = kNegBig;
    for (int i = 0; i < kWave; ++i) M = fmaxf(M, ml[i][0]);
    const float f = fast_exp2(m - M);
#pragma unroll
    for (int d = 0; d < D; ++d) part[lane][d] = o[d] * f;
    __syncthreads();
    float den = 0.f;
    for (int i = 0; i < kWave; ++i) den += ml[i][1] * fast_exp2(ml[i][0] - M);
    for (int d = lane; d < D; d += kWave) {
        float acc = 0.f;
        for (int i = 0; i < kWave; ++i) acc += part[i][d];
        orow[d] = acc / den;
    }
}

int env_int(const char *name, int dflt) {
    const char *v = getenv(name);
    return (v && *v) ? atoi(v) : dflt;
}

}  // namespace

AttnPlan plan_attention(int dtype, int B, int P_max, int Hq, int Hkv, int D, int S_max) {
    AttnPlan plan{0, 1, kBlockN, 0};
    if (dtype != 1) return plan;  // fp32 path needs no workspace
    const int G = Hq / Hkv;
    plan.nqblk = (G * P_max + kBlockM - 1) / kBlockM;
    // Split the cache only as far as needed for about four workgroups per
    // CU, and never below 16 key tiles (1024 keys) per split: shorter
    // splits spend more on partial writes and the merge than they gain in
    // parallelism (measured on MI355X).
    const long units = static_cast<long>(B) * Hkv * plan.nqblk;
    const int tiles = (S_max + kBlockN - 1) / kBlockN;
    const long target = 4L * device_cu_count();
    int nsplit = static_cast<int>((target + units - 1) / units);
    nsplit = min(nsplit, max(1, tiles / 16));
    nsplit = env_int("RD_ATTN_SPLITS", nsplit);
    nsplit = max(1, min(nsplit, min(max(tiles, 1), kMaxSplits)));
    const int chunk_tiles = (max(tiles, 1) + nsplit - 1) / nsplit;
    plan.nsplit = (max(tiles, 1) + chunk_tiles - 1) / chunk_tiles;
    plan.chunk = chunk_tiles * kBlockN;
    if (plan.nsplit > 1) {
        const size_t rows = static_cast<size_t>(B) * Hkv * plan.nsplit * plan.nqblk * kBlockM;
        plan.ws_bytes = rows * (static_cast<size_t>(D) * sizeof(float) + sizeof(float2));
    }
    return plan;
}

hipError_t launch_attention(int dtype, const AttnPlan &plan, const void *q, const void *k_new,
                            const void *v_new, const void *k_cache, const void *v_cache,
                            const int32_t *kv_len, const uint32_t *mask, const int32_t *plen, int B,
                            int P_max, int Hq, int Hkv, int D, int S_max, float scale, void *out,
                            void *ws, hipStream_t stream) {
    const float sc = (scale == 0.f) ? 1.f / sqrtf(static_cast<float>(D)) : scale;
    const int nw = (P_max + 31) / 32;
    if (dtype == 0) {
        const dim3 grid(static_cast<unsigned>(static_cast<size_t>(B) * P_max * Hq));
        auto kern = (D == 64) ? k_tree_attn_f32<64> : k_tree_attn_f32<128>;
        hipLaunchKernelGGL(kern, grid, dim3(kWave), 0, stream, static_cast<const float *>(q),
                           static_cast<const float *>(k_new), static_cast<const float *>(v_new),
                           static_cast<const float *>(k_cache), static_cast<const float *>(v_cache), kv_len,
                           mask, plen, P_max, Hq, Hkv, S_max, nw, sc * kLog2e, static_cast<float *>(out));
        return hipGetLastError();
    }
    AttnArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k_new = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.k_cache = static_cast<const uint16_t *>(k_cache);
    a.v_cache = static_cast<const uint16_t *>(v_cache);
    a.kv_len = kv_len;
    a.mask = mask;
    a.plen = plen;
    a.B = B;
    a.P = P_max;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.S_max = S_max;
    a.nw = nw;
    a.scale_log2 = sc * kLog2e;
    a.nqblk = plan.nqblk;
    a.nsplit = plan.nsplit;
    a.chunk = plan.chunk;
    a.out = static_cast<uint16_t *>(out);
    const size_t rows = static_cast<size_t>(B) * Hkv * plan.nsplit * plan.nqblk * kBlockM;
    a.ws_o = static_cast<float *>(ws);
    a.ws_ml = (plan.nsplit > 1) ? reinterpret_cast<float2 *>(static_cast<float *>(ws) + rows * D) : nullptr;
    const unsigned nblk = static_cast<unsigned>(static_cast<size_t>(B) * Hkv * plan.nsplit * plan.nqblk);
    if (D == 64)
        hipLaunchKernelGGL(k_tree_attn_bf16<64>, dim3(nblk), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(k_tree_attn_bf16<128>, dim3(nblk), dim3(256), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || plan.nsplit == 1) return err;
    const unsigned ncomb = static_cast<unsigned>(static_cast<size_t>(B) * Hkv * plan.nqblk);
    if (D == 64)
        hipLaunchKernelGGL(k_attn_combine<64>, dim3(ncomb), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(k_attn_combine<128>, dim3(ncomb), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rd
