// Step 2: tree attention over the packed tokens.
//
// ReDrafter verifies every candidate path of the beam tree in one pass
// (TensorRT-LLM ReDrafter blog, intro and FAQ; Apple/NVIDIA news article,
// "Dynamic tree attention").  Packed query p attends to all cached keys of
// its request and to the packed keys whose bit is set in its tree-mask row
// (SpecInfer's topology-aware causal mask, speculative-decoding survey,
// "Token Tree Verifier").
//
// bf16 kernel layout.  One workgroup (4 wavefronts) handles up to RB query
// rows of one (request, KV head) and one split of the KV cache; row r of the
// (request, KV head) is packed token r / G, query head g*G + r % G, so the G
// heads sharing a KV head share every K/V tile, and all rows of a (request,
// KV head) normally sit in one workgroup, so the cache is streamed once.
// Keys stream through LDS in tiles of 64: cache tiles first, then (last
// split only) the packed tiles up to the largest token of the block --
// parents precede children, so later tokens cannot be ancestors.
//
// K and V tiles are copied global->LDS by direct loads (whole cache lines,
// no registers) into a ring of NS stages, in their natural [key][d] layout
// with 16-byte chunks XOR-swizzled by key.  Scores are computed transposed,
// S^T = K Q^T (A = K rows, B = Q held in registers), so each lane's
// accumulator column is one query and the probabilities P^T come out of the
// MFMA already in the B-operand layout of O^T = V^T P^T.  The V^T operand
// is read with the gfx950 LDS transpose load (ds_read_b64_tr_b16), which
// turns a 16-lane group's 16 x 4 block into 4 consecutive keys per lane.
// Each wavefront owns up to QPW blocks of 16 query rows and reuses every
// K and V fragment it reads across them.  Online softmax runs in fp32 in
// the log2 domain.  With more than one split, each split writes (max, sum,
// unnormalised O) in fp32 and a combine kernel merges them.
#include <math.h>
#include <stdlib.h>

#include "rd_common.h"
#include "rd_internal.h"

namespace rd {

namespace {

constexpr int kBlockN = 64;  // keys per tile
constexpr int kCombRows = 64;  // rows per combine workgroup
constexpr int kMaxSplits = 64;
constexpr int kMaxMaskWords = (kMaxBeams * kMaxBeamLen) / 32;
constexpr int kStages = 3;
constexpr float kRescale = 8.f;  // lazy-rescale threshold of the online softmax (log2 units)

struct AttnArgs {
    const uint16_t *q, *k_new, *v_new, *k_cache, *v_cache;
    const int32_t *kv_len;
    const uint32_t *mask;
    const int32_t *plen;
    int B, P, Hq, Hkv, G, S_max, nw;
    float scale_log2;
    int nqblk, nsplit, chunk, rows_unit;  // rows_unit = nqblk * rows per workgroup
    uint16_t *out;
    float *ws_o;    // [B, Hkv, nsplit, rows_unit, D]
    float2 *ws_ml;  // [B, Hkv, nsplit, rows_unit]
};

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// LDS transpose load: within each 16-lane group, lane i receives element
// i % 4 of the 4-element rows addressed by lanes i/4, i/4 + 4, i/4 + 8 and
// i/4 + 12 (lane layout established on gfx950).
__device__ __forceinline__ bf16x4 lds_read_tr16(uint32_t addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<lds_bf16x4 *>(static_cast<uintptr_t>(addr)));
}

template <int D, int QPW, int NWAVE>
__global__ __launch_bounds__(64 * NWAVE, 1) void k_tree_attn_bf16(AttnArgs a) {
    constexpr int NKC = D / 32;              // k-steps over the head dim (QK^T)
    constexpr int NDB = D / 16;              // 16-row blocks of the head dim (PV)
    constexpr int KCH = D / 8;               // 16-byte chunks per key row
    constexpr int ROWB = D * 2;              // bytes per key row
    constexpr int TILEB = kBlockN * ROWB;    // bytes of one K or V tile
    constexpr int STAGEB = 2 * TILEB;        // K tile then V tile
    constexpr int KPL = 1024 / ROWB;         // keys per 1 KB load instruction
    constexpr int NT = 64 * NWAVE;           // threads per workgroup
    constexpr int NLD = kBlockN / KPL / NWAVE;  // load instructions per wavefront per operand per tile
    constexpr int RB = NWAVE * QPW * 16;     // query rows per workgroup
    static_assert(NLD >= 1, "every wavefront issues loads");
    static_assert(KCH >= 8, "the swizzle permutes 8 chunks");
    __shared__ __attribute__((aligned(1024))) uint8_t stage[kStages * STAGEB];
    __shared__ uint32_t mwords[RB * kMaxMaskWords];  // tree-mask rows of this block's tokens

    // row blocks are the slowest index: blocks with no valid rows (their
    // count depends on the packed lengths) come last in dispatch order
    const int L = a.B * a.Hkv * a.nsplit;
    const int qb = blockIdx.x / L;
    const int rest = blockIdx.x - qb * L;
    const int s = rest % a.nsplit;
    const int g = (rest / a.nsplit) % a.Hkv;
    const int b = rest / (a.nsplit * a.Hkv);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 15;
    const int kg = lane >> 4;

    const int Pb = min(max(a.plen[b], 0), a.P);
    const int kvl = min(max(a.kv_len[b], 0), a.S_max);
    const int Mb = a.G * Pb;
    const int Mpad = a.G * a.P;
    const int row0 = qb * RB;

    if (row0 >= Mb) {
        // no valid query rows: with a single split this block owns the
        // padding rows of the output and writes them as zeros
        if (a.nsplit == 1) {
            for (int i = tid; i < RB * KCH; i += NT) {
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
        tok_hi = (min(row0 + RB, Mb) - 1) / a.G + 1;
        npk = (tok_hi + kBlockN - 1) / kBlockN;
    }
    const int ntile = ncache + npk;
    const int tok_lo = row0 / a.G;

    // this lane's query rows: block qi of wavefront w covers rows
    // row0 + (NWAVE*qi + w)*16 .. +15 (interleaved, so few rows still
    // spread over the wavefronts)
    // A wavefront with at least one valid row multiplies all its blocks
    // (padding rows hold zero queries); one with none only helps with the
    // loads.  Valid rows form a prefix, so block 0 decides.
    bf16x8 qf[QPW][NKC];
    int lt[QPW];  // token of the row relative to tok_lo
    const bool wave_active = row0 + wave * 16 < Mb;
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
        const int r = row0 + (NWAVE * qi + wave) * 16 + lq;
        const bool rvalid = r < Mb;
        const int p = rvalid ? r / a.G : 0;
        const int h = g * a.G + (rvalid ? r % a.G : 0);
        lt[qi] = rvalid ? p - tok_lo : 0;
        const uint16_t *qrow = a.q + ((static_cast<size_t>(b) * a.P + p) * a.Hq + h) * D;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
            qf[qi][kc] = as_bf16x8(rvalid ? ld16(qrow + 32 * kc + 8 * kg) : make_uint4(0, 0, 0, 0));
    }
    // tokens of this block and their tree-mask rows, staged in LDS once
    if (npk > 0) {
        const int ntok = tok_hi - tok_lo;
        const uint32_t *msrc = a.mask + (static_cast<size_t>(b) * a.P + tok_lo) * a.nw;
        for (int i = tid; i < ntok * a.nw; i += NT) mwords[i] = msrc[i];
    }
    // The Q loads must land before the ring starts: at a first use inside
    // the loop the compiler would wait for them -- and thereby for every ring
    // load issued after them.
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi)
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) asm volatile("" : "+v"(qf[qi][kc]));

    // K/V rows of tile i: cache tiles come first, then the packed tiles.
    // Keys past the valid range get an out-of-range offset and load zeros.
    const size_t cache_base = (static_cast<size_t>(b) * a.Hkv + g) * a.S_max * D;
    const size_t fresh_base = (static_cast<size_t>(b) * a.P * a.Hkv + g) * D;
    const uint32_t cache_bytes = static_cast<uint32_t>(min<size_t>(static_cast<size_t>(a.S_max) * D * 2, kMaxRange));
    const uint32_t fresh_bytes = static_cast<uint32_t>(min<size_t>(static_cast<size_t>(a.P) * a.Hkv * D * 2, kMaxRange));
    const i32x4_t rk_c = make_srsrc(a.k_cache + cache_base, cache_bytes);
    const i32x4_t rv_c = make_srsrc(a.v_cache + cache_base, cache_bytes);
    const i32x4_t rk_n = make_srsrc(a.k_new + fresh_base, fresh_bytes);
    const i32x4_t rv_n = make_srsrc(a.v_new + fresh_base, fresh_bytes);
    const uint32_t lds0 = lds_addr_of(stage);

    // Cache tiles are visited from a per-block starting tile (wrapping) so
    // that concurrent blocks, whose slabs sit at power-of-two strides, do
    // not all address the same offsets and crowd a few HBM channels.
    const int trot = ncache > 0 ? (b * 7 + g * 3 + qb * 5) % ncache : 0;
    // Load j = NWAVE*jj + wave of an operand covers tile keys KPL*j .. +KPL-1;
    // lane i stores LDS chunk slot i % KCH of key KPL*j + i / KCH, which
    // holds head-dim chunk slot ^ (key & 7).
    const int lkey = lane / KCH;
    const int lslot = lane % KCH;
    auto issue_tile = [&](int i, int slot) {
        const bool cache = i < ncache;
        const i32x4_t rk = cache ? rk_c : rk_n;
        const i32x4_t rv = cache ? rv_c : rv_n;
        const int ic = (i + trot >= ncache) ? i + trot - ncache : i + trot;
        const int kbase = cache ? c0 + ic * kBlockN : (i - ncache) * kBlockN;
        const int klim = (i >= ntile) ? 0 : (cache ? c1 : tok_hi);
        const uint32_t rowstride = cache ? ROWB : static_cast<uint32_t>(a.Hkv) * ROWB;
        const uint32_t kdst = lds0 + slot * STAGEB;
#pragma unroll
        for (int jj = 0; jj < NLD; ++jj) {
            const int j = NWAVE * jj + wave;
            const int kl = KPL * j + lkey;
            const int key = kbase + kl;
            const uint32_t off = key < klim ? static_cast<uint32_t>(key) * rowstride + ((lslot ^ (kl & 7)) << 4) : kOOB;
            lds_dma16(kdst + j * 1024, rk, off);
            lds_dma16(kdst + TILEB + j * 1024, rv, off);
        }
    };

    // fragment offsets within a stage (see the swizzle above)
    uint32_t koff[NKC];  // K row (kb*16 + lq), chunk 4*kc + kg; add kb*16*ROWB
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) koff[kc] = lq * ROWB + (((4 * kc + kg) ^ (lq & 7)) << 4);
    // V^T: 16-lane group kg reads keys base + 4*kg + j/4 (j = lane % 16),
    // head dims 16*db + 4*(j%4) .. +3; chunk 2*db + (j%4)/2, half (j%4)&1
    const int vj = lane & 15;
    const int vkey = 4 * kg + (vj >> 2);
    const int vsw = vkey & 7;
    uint32_t voff[4];  // for db & 3; chunk bit 3 (db >> 2) is not swizzled: +128 bytes
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) {
        const int chunk = 2 * d4 + ((vj & 3) >> 1);
        voff[d4] = TILEB + vkey * ROWB + ((chunk ^ vsw) << 4) + ((vj & 1) << 3);
    }

    f32x4 o[QPW][NDB];
    float mrun[QPW], lpart[QPW];
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[qi][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        mrun[qi] = kNegBig;
        lpart[qi] = 0.f;
    }

    // One pass over the tile for query blocks q0 .. q0+QG-1.
    constexpr int QG = QPW < 2 ? QPW : 2;
    auto compute_group = [&](int i, uint32_t sbase, int q0) {
        const uint8_t *st = stage + (sbase - lds0);
        // S^T for 64 keys x 16 queries per block; the K fragments of a
        // head-dim step are read once (one step ahead) for all blocks of the
        // pass.  Scores stay unscaled: the scale folds into the exponent.
        f32x4 sc[QG][4];
#pragma unroll
        for (int qi = 0; qi < QG; ++qi)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sc[qi][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 ka[2][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) ka[0][kb] = *reinterpret_cast<const bf16x8 *>(st + koff[0] + kb * 16 * ROWB);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            if (kc + 1 < NKC)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    ka[(kc + 1) & 1][kb] = *reinterpret_cast<const bf16x8 *>(st + koff[kc + 1] + kb * 16 * ROWB);
#pragma unroll
            for (int qi = 0; qi < QG; ++qi)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    sc[qi][kb] = mfma16x16x32(ka[kc & 1][kb], qf[q0 + qi][kc], sc[qi][kb]);
        }

        // mask (partial cache tiles and packed tiles only), online softmax;
        // key of sc[qi][kb][e] within the tile is kb*16 + 4*kg + e
        const bool cache = i < ncache;
        const int ic = (i + trot >= ncache) ? i + trot - ncache : i + trot;
        const int lim = cache ? c1 - (c0 + ic * kBlockN) : tok_hi - (i - ncache) * kBlockN;
        const bool full = cache && lim >= kBlockN;  // wave-uniform
        const int wi = 2 * (i - ncache);
        if (!full) {
#pragma unroll
            for (int qi = 0; qi < QG; ++qi) {
                uint32_t w0 = 0xffffffffu, w1 = 0xffffffffu;
                if (!cache) {
                    w0 = mwords[lt[q0 + qi] * a.nw + wi];
                    w1 = (wi + 1 < a.nw) ? mwords[lt[q0 + qi] * a.nw + wi + 1] : 0u;
                }
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = kb * 16 + 4 * kg + e;
                        const uint32_t wd = (j < 32) ? w0 : w1;
                        const bool vis = (j < lim) && ((wd >> (j & 31)) & 1u);
                        sc[qi][kb][e] = vis ? sc[qi][kb][e] : -INFINITY;
                    }
            }
        }
        bf16x8 pb[QG][2];
#pragma unroll
        for (int qi = 0; qi < QG; ++qi) {
            const int q = q0 + qi;
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, sc[qi][kb][e]);
            tmax = fmaxf(tmax, shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, shfl_xor(tmax, 32));
            tmax *= a.scale_log2;  // the scale is positive
            // Lazy rescale: the reference max moves only when some row's max
            // has grown by more than kRescale (log2 units), so O and l stay
            // in registers untouched on most tiles.  Exact: O and l are both
            // taken relative to the same reference, and probabilities stay
            // below 2^kRescale.
            if (__any(tmax > mrun[q] + kRescale)) {
                const float mnew = fmaxf(mrun[q], tmax);
                const float alpha = fast_exp2(mrun[q] - mnew);
                mrun[q] = mnew;
                lpart[q] *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[q][db] *= alpha;
            }
            const float mref = mrun[q];
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sc[qi][kb][e] = fast_exp2(fmaf(sc[qi][kb][e], a.scale_log2, -mref));
                    psum += sc[qi][kb][e];
                }
            lpart[q] += psum;
            // P^T as the B operand of the two 32-key steps: slots 0-3 hold
            // keys 32*ks + 4*kg + (0..3), slots 4-7 keys 32*ks + 16 + 4*kg + (0..3)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pb[qi][ks][e] = static_cast<__bf16>(sc[qi][2 * ks][e]);
                    pb[qi][ks][4 + e] = static_cast<__bf16>(sc[qi][2 * ks + 1][e]);
                }
        }

        // O^T += V^T P^T over 2*NDB steps (ks, db); each V^T fragment (two
        // transpose loads) serves every block of the pass and is read kVPre
        // steps ahead
        constexpr int NSTEP = 2 * NDB;
        constexpr int kVPre = 4;
        auto vaddr = [&](int n) {
            const int ks = n / NDB, db = n % NDB;
            return sbase + voff[db & 3] + (db >> 2) * 128 + ks * 32 * ROWB;
        };
        bf16x4 vlo[kVPre], vhi[kVPre];
#pragma unroll
        for (int n = 0; n < kVPre; ++n) {
            vlo[n] = lds_read_tr16(vaddr(n));
            vhi[n] = lds_read_tr16(vaddr(n) + 16 * ROWB);
        }
#pragma unroll
        for (int n = 0; n < NSTEP; ++n) {
            bf16x8 vf;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vf[e] = vlo[n % kVPre][e];
                vf[4 + e] = vhi[n % kVPre][e];
            }
            if (n + kVPre < NSTEP) {
                vlo[n % kVPre] = lds_read_tr16(vaddr(n + kVPre));
                vhi[n % kVPre] = lds_read_tr16(vaddr(n + kVPre) + 16 * ROWB);
            }
            const int ks = n / NDB, db = n % NDB;
#pragma unroll
            for (int qi = 0; qi < QG; ++qi) o[q0 + qi][db] = mfma16x16x32(vf, pb[qi][ks], o[q0 + qi][db]);
        }
    };
    auto compute_tile = [&](int i, uint32_t sbase) {
#pragma unroll
        for (int q0 = 0; q0 < QPW; q0 += QG) compute_group(i, sbase, q0);
    };

    // Ring of kStages LDS stages.  Tiles 0..kStages-2 are issued up front.
    // At the top of tile i this wavefront's loads of tile i have landed once
    // at most (kStages-2)*2*NLD of its loads remain outstanding; the barrier
    // publishes every wavefront's share and certifies that all reads of the
    // slot of tile i-1 are done, so tile i+kStages-1 may be loaded into it.
    // Tiles past the last still issue their loads, all out of range, so
    // every wait counts the same number of loads.
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st) issue_tile(st, st);
    int cslot = 0, lslot_ring = kStages - 1;  // slots of the tile computed / loaded
    for (int i = 0; i < ntile; ++i) {
        vm_wait<(kStages - 2) * 2 * NLD>();
        __syncthreads();
        issue_tile(i + kStages - 1, lslot_ring);
        if (wave_active) compute_tile(i, lds0 + cslot * STAGEB);
        cslot = (cslot + 1 == kStages) ? 0 : cslot + 1;
        lslot_ring = (lslot_ring + 1 == kStages) ? 0 : lslot_ring + 1;
    }
    vm_wait<0>();

#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
        float lsum = lpart[qi] + shfl_xor(lpart[qi], 16);
        lsum += shfl_xor(lsum, 32);
        const int r = row0 + (NWAVE * qi + wave) * 16 + lq;
        const bool rvalid = r < Mb;
        if (a.nsplit == 1) {
            // o[qi][db][e] = O[query r][d = db*16 + 4*kg + e]; padding rows get zeros
            if (r < Mpad) {
                const float inv = (rvalid && lsum > 0.f) ? 1.f / lsum : 0.f;
                const int pz = r / a.G, hz = g * a.G + r % a.G;
                uint16_t *orow = a.out + ((static_cast<size_t>(b) * a.P + pz) * a.Hq + hz) * D;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    u16x4 w = {f32_to_bf16_bits(o[qi][db][0] * inv), f32_to_bf16_bits(o[qi][db][1] * inv),
                               f32_to_bf16_bits(o[qi][db][2] * inv), f32_to_bf16_bits(o[qi][db][3] * inv)};
                    *reinterpret_cast<u16x4 *>(orow + db * 16 + 4 * kg) = w;
                }
            }
        } else if (rvalid) {
            const size_t prow = ((static_cast<size_t>(b) * a.Hkv + g) * a.nsplit + s) * a.rows_unit + r;
            float *orow = a.ws_o + prow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4 *>(orow + db * 16 + 4 * kg) = o[qi][db];
            if (kg == 0) a.ws_ml[prow] = make_float2(mrun[qi], lsum);
        }
    }
}

// Merge of the per-split partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
    constexpr int KCH4 = D / 4;  // float4 chunks per row
    __shared__ float wgt[kCombRows][kMaxSplits + 1];
    const int nrb = a.rows_unit / kCombRows;
    const int qb = blockIdx.x % nrb;
    const int bg = blockIdx.x / nrb;
    const int g = bg % a.Hkv;
    const int b = bg / a.Hkv;
    const int Pb = min(max(a.plen[b], 0), a.P);
    const int Mb = a.G * Pb;
    const int Mpad = a.G * a.P;
    const int row0 = qb * kCombRows;
    const size_t split_stride = static_cast<size_t>(a.rows_unit);
    const size_t base = (static_cast<size_t>(b) * a.Hkv + g) * a.nsplit * split_stride;

    if (threadIdx.x < kCombRows) {
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
    for (int i = threadIdx.x; i < kCombRows * KCH4; i += 256) {
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
    AttnPlan plan{0, 1, kBlockN, 0, 1, 0, 4};
    if (dtype != 1) return plan;  // fp32 path needs no workspace
    const int G = Hq / Hkv;
    const int rows = G * P_max;
    // 16-row query blocks per wavefront: enough that one workgroup holds all
    // rows of a (request, KV head) whenever they fit in 256
    // (QPW, wavefronts) = (1, 4), (2, 4) or (2, 8): 64, 128 or 256 rows
    plan.qpw = rows <= 64 ? 1 : 2;
    plan.nwave = rows <= 128 ? 4 : 8;
    const int rb = 16 * plan.qpw * plan.nwave;
    plan.nqblk = (rows + rb - 1) / rb;
    plan.rows_unit = plan.nqblk * rb;
    // One workgroup per CU fits (the LDS ring): split the cache only as far
    // as needed to give every CU a workgroup, and never below 8 key tiles
    // per split.
    const long units = static_cast<long>(B) * Hkv * plan.nqblk;
    const int tiles = (S_max + kBlockN - 1) / kBlockN;
    const long target = device_cu_count();
    int nsplit = static_cast<int>((target + units - 1) / units);
    nsplit = min(nsplit, max(1, tiles / 8));
    nsplit = env_int("RD_ATTN_SPLITS", nsplit);
    nsplit = max(1, min(nsplit, min(max(tiles, 1), kMaxSplits)));
    const int chunk_tiles = (max(tiles, 1) + nsplit - 1) / nsplit;
    plan.nsplit = (max(tiles, 1) + chunk_tiles - 1) / chunk_tiles;
    plan.chunk = chunk_tiles * kBlockN;
    if (plan.nsplit > 1) {
        const size_t nrow = static_cast<size_t>(B) * Hkv * plan.nsplit * plan.rows_unit;
        plan.ws_bytes = nrow * (static_cast<size_t>(D) * sizeof(float) + sizeof(float2));
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
    a.rows_unit = plan.rows_unit;
    a.out = static_cast<uint16_t *>(out);
    const size_t nrow = static_cast<size_t>(B) * Hkv * plan.nsplit * plan.rows_unit;
    a.ws_o = static_cast<float *>(ws);
    a.ws_ml = (plan.nsplit > 1) ? reinterpret_cast<float2 *>(static_cast<float *>(ws) + nrow * D) : nullptr;
    const dim3 grid(static_cast<unsigned>(static_cast<size_t>(B) * Hkv * plan.nsplit * plan.nqblk));
    const dim3 blk(64 * plan.nwave);
    if (D == 64) {
        if (plan.qpw == 1) hipLaunchKernelGGL((k_tree_attn_bf16<64, 1, 4>), grid, blk, 0, stream, a);
        else if (plan.nwave == 4) hipLaunchKernelGGL((k_tree_attn_bf16<64, 2, 4>), grid, blk, 0, stream, a);
        else hipLaunchKernelGGL((k_tree_attn_bf16<64, 2, 8>), grid, blk, 0, stream, a);
    } else {
        if (plan.qpw == 1) hipLaunchKernelGGL((k_tree_attn_bf16<128, 1, 4>), grid, blk, 0, stream, a);
        else if (plan.nwave == 4) hipLaunchKernelGGL((k_tree_attn_bf16<128, 2, 4>), grid, blk, 0, stream, a);
        else hipLaunchKernelGGL((k_tree_attn_bf16<128, 2, 8>), grid, blk, 0, stream, a);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || plan.nsplit == 1) return err;
    const unsigned ncomb = static_cast<unsigned>(static_cast<size_t>(B) * Hkv * (plan.rows_unit / kCombRows));
    if (D == 64)
        hipLaunchKernelGGL(k_attn_combine<64>, dim3(ncomb), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(k_attn_combine<128>, dim3(ncomb), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rd
