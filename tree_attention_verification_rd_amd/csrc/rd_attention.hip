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

#include <type_traits>

#include "../../include/rd.h"
#include "rd_common.h"
#include "rd_internal.h"

namespace rd {

namespace {

constexpr int kBlockN = 64;  // keys per tile
constexpr int kCombRows = 64;  // rows per combine workgroup
constexpr int kMaxSplits = 64;
constexpr int kMaxMaskWords = (kMaxBeams * kMaxBeamLen) / 32;
constexpr float kRescale = 8.f;  // lazy-rescale threshold of the online softmax (log2 units)
constexpr int kTileFull = 0, kTileMasked = 1;  // kinds of key tile

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
    // paged cache: k_cache / v_cache are pools [num_pages, Hkv, page_size, D]
    const int32_t *bt;  // block table [B, max_pages]
    int max_pages, page_size;
    int64_t num_pages;
};

typedef const int32_t __attribute__((address_space(4))) cint32_t;  // read through the scalar cache

// Page of logical cache position t of request b (clamped into the pool).
__device__ __forceinline__ int64_t page_of(const AttnArgs &a, int b, int t) {
    const int32_t pg = ((cint32_t *)a.bt)[static_cast<size_t>(b) * a.max_pages + t / a.page_size];
    return min(max(static_cast<int64_t>(pg), static_cast<int64_t>(0)), a.num_pages - 1);
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// Maximum over lanes i, i^16, i^32 and i^48 (the four k-groups of an MFMA
// output column), without LDS: v_permlane32_swap (v_permlane16_swap) with
// both operands t leaves t of lanes i and i^32 (i^16) in its two results.
__device__ __forceinline__ float max_over_kgroups(float t) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    t = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    return fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
}

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
typedef __attribute__((address_space(3))) uint8_t lds_u8;
// the same read from an LDS byte pointer: a constant added to a common base
// folds into the instruction's offset field instead of an address add
__device__ __forceinline__ bf16x4 lds_read_tr16(const lds_u8 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<lds_bf16x4 *>(const_cast<lds_u8 *>(p)));
}

// Rows of query block qi of query group q: blocked, rows row0 + (NQG*qi +
// q)*16 + (0..15), or, with LI (lane-interleaved, for few rows), rows
// row0 + (16*qi + j)*NQG + q for lane j, so a handful of rows still gives
// every query group -- and so every wavefront -- work.
// With PAGED the cache comes from a page pool: the page size is a multiple
// of the 64-key tile, so each cache tile lies in one page, and the tile's
// load resource starts at that page's rows for this KV head.
template <int D, int QPW, int NWAVE, int KSPLIT, int NS, bool LI, bool PAGED>
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
    constexpr int NQG = NWAVE / KSPLIT;      // query groups (wavefronts per key group)
    constexpr int RB = NQG * QPW * 16;       // query rows per workgroup
    constexpr int KW = kBlockN / KSPLIT;     // keys of a tile per key group
    constexpr int NKB = KW / 16;             // 16-key blocks per key group
    constexpr int NKS = KW / 32;             // 32-key PV steps per key group
    static_assert(NLD >= 1, "every wavefront issues loads");
    static_assert(KCH >= 8, "the swizzle permutes 8 chunks");
    static_assert(QPW == 1 || QPW == 2, "one or two query blocks per wavefront");
    static_assert(KSPLIT == 1 || KSPLIT == 2, "a tile's keys go to one or two key groups");
    __shared__ __attribute__((aligned(1024))) uint8_t stage[NS * STAGEB];
    __shared__ uint32_t mwords[RB * kMaxMaskWords];  // tree-mask rows of this block's tokens

    // Row blocks are the slowest index: blocks with no valid rows (their
    // count depends on the packed lengths) come last in dispatch order.
    // Interleaving them with real blocks -- e.g. to run the two row blocks
    // of one (request, KV head) side by side on one XCD so that the second
    // cache read hits L2 -- measured up to 1.8x slower (gqa, dedup sweep at
    // p = 0.9): the idle blocks' places in the dispatch order leave some
    // shader engines with most of the real work.
    const int L_ = a.B * a.Hkv * a.nsplit;
    const int qb = blockIdx.x / L_;
    const int rest = blockIdx.x - qb * L_;
    const int s = rest % a.nsplit;
    const int g = (rest / a.nsplit) % a.Hkv;
    const int b = rest / (a.nsplit * a.Hkv);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wq = wave % NQG;  // query group
    const int wk = wave / NQG;  // key group: keys wk*KW .. wk*KW+KW-1 of every tile
    const int lane = tid & 63;
    const int lq = lane & 15;
    const int kg = lane >> 4;
    auto row_of = [&](int qi, int j) {  // row of lane slot j in this group's block qi, relative to row0
        return LI ? (16 * qi + j) * NQG + wq : (NQG * qi + wq) * 16 + j;
    };

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
    // values the lambdas below read are const: a mutable local selected by
    // reference in a lambda stays in scratch memory
    const int tok_hi = (s == a.nsplit - 1) ? (min(row0 + RB, Mb) - 1) / a.G + 1 : 0;
    const int npk = (tok_hi + kBlockN - 1) / kBlockN;
    const int ntile = ncache + npk;
    const int tok_lo = row0 / a.G;
    bf16x8 qf[QPW][NKC];
    int lt[QPW];  // token of the row relative to tok_lo
    int nact = 0;

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

    // Cache tile i holds the split's keys c0 + pos(j), j = 0..63, with
    // pos(j) = ic*64 + j, or, on the split-KV path, the strided ic + ncache*j
    // (the cache part of the softmax does not depend on key order; strided
    // tiles spread each load of a long cache over many HBM pages instead of
    // one 16 KB run, which measured faster there and slower elsewhere).  ic
    // is rotated per (request, KV head) so that concurrent blocks, whose
    // slabs sit at power-of-two strides, do not all address the same
    // offsets; the row blocks of one (request, KV head) share the rotation.
    const int nck = c1 - c0;  // cache keys of this split
    const bool strided = !PAGED && a.nsplit > 1;
    const int kmul = strided ? ncache : 1;  // pos(j) = ic*kblk + kmul*j
    const int kblk = strided ? 1 : kBlockN;
    // Tiles ic < nfull are full (every key before the split's end), the
    // rest of the cache tiles partial.  The rotation runs over the full
    // tiles only, so the partial ones come after them and the loop splits
    // into a run of full tiles and a run of masked ones (partial cache tiles,
    // then packed tiles).
    const int nfull = strided ? min(max(nck - (kBlockN - 1) * ncache, 0), ncache) : nck / kBlockN;
    const int trot = nfull > 0 ? (b * 7 + g * 3) % nfull : 0;  // the same for every row block
    auto tile_ic = [=](int i) { return i < nfull ? (i + trot >= nfull ? i + trot - nfull : i + trot) : i; };
    // Load j = NWAVE*jj + wave of an operand covers tile keys KPL*j .. +KPL-1;
    // lane i stores LDS chunk slot i % KCH of key KPL*j + i / KCH, which
    // holds head-dim chunk slot ^ (key & 7).
    const int lkey = lane / KCH;
    const int lslot = lane % KCH;
    const int c1v = c1;
    // by value: a closure holding references to these locals kept them in
    // scratch memory and selected between their addresses
    auto issue_tile = [=](int i, int slot) {
        const bool cache = i < ncache;
        i32x4_t rk = cache ? rk_c : rk_n;
        i32x4_t rv = cache ? rv_c : rv_n;
        const int ic = tile_ic(i);
        const int kbase = cache ? c0 + ic * kblk : (i - ncache) * kBlockN;
        const int klim = (i >= ntile) ? 0 : (cache ? c1v : tok_hi);
        const uint32_t rowstride = cache ? ROWB : static_cast<uint32_t>(a.Hkv) * ROWB;
        const uint32_t kdst = lds0 + slot * STAGEB;
        int kres = 0;  // key at the resource base
        if constexpr (PAGED) {
            if (cache) {
                const int64_t pg = page_of(a, b, kbase);
                const size_t e0 = ((static_cast<size_t>(pg) * a.Hkv + g) * a.page_size + kbase % a.page_size) * D;
                rk = make_srsrc(a.k_cache + e0, TILEB);
                rv = make_srsrc(a.v_cache + e0, TILEB);
                kres = kbase;
            }
        }
        // Lane offsets from the tile's first key: kk keys and, to the lane's
        // chunk, lo bytes -- keys kmul apart in rows of ROWB bytes for a cache
        // tile, consecutive keys in rows of Hkv*ROWB bytes for a packed one.
        // Both forms are loop-invariant values (hoisted), so a tile's loads
        // select between them and multiply nothing.
        const int krem = klim - kbase;  // keys kbase + kk with kk < krem are in range
        const uint32_t obase = static_cast<uint32_t>(kbase - kres) * rowstride;
#pragma unroll
        for (int jj = 0; jj < NLD; ++jj) {
            const int j = NWAVE * jj + wave;
            const int kl = KPL * j + lkey;
            const uint32_t sw = static_cast<uint32_t>(lslot ^ (kl & 7)) << 4;
            const int kk_c = kmul * kl;
            const uint32_t lo_c = static_cast<uint32_t>(kk_c) * ROWB + sw;
            const uint32_t lo_n = static_cast<uint32_t>(kl) * (static_cast<uint32_t>(a.Hkv) * ROWB) + sw;
            const int kk = cache ? kk_c : kl;
            const uint32_t off = kk < krem ? obase + (cache ? lo_c : lo_n) : kOOB;
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

    // The stages of one tile, for query blocks 0 .. NQ-1 (NQ from the
    // arrays' extent).  qk_scores: S^T = K Q^T; K fragments of a head-dim
    // step are read one step ahead and serve every block; scores stay
    // unscaled (the scale folds into the exponent).
    auto qk_scores = [&](uint32_t sbase, auto &sc) {
        constexpr int NQ = sizeof(sc) / sizeof(sc[0]);
        const uint8_t *st = stage + (sbase - lds0);
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) sc[qi][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint32_t kgrp = wk * NKB * 16 * ROWB;
        bf16x8 ka[2][NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            ka[0][kb] = *reinterpret_cast<const bf16x8 *>(st + kgrp + koff[0] + kb * 16 * ROWB);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            if (kc + 1 < NKC)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    ka[(kc + 1) & 1][kb] = *reinterpret_cast<const bf16x8 *>(st + kgrp + koff[kc + 1] + kb * 16 * ROWB);
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) sc[qi][kb] = mfma16x16x32(ka[kc & 1][kb], qf[qi][kc], sc[qi][kb]);
        }
    };
    // maxima of a tile's scores in log2 units over each lane's own keys of
    // its row (the row maximum is the largest of its four k-groups' values)
    auto tile_max = [&](const auto &sc, float *tmax) {
        constexpr int NQ = sizeof(sc) / sizeof(sc[0]);
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            float t = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) t = fmaxf(t, sc[qi][kb][e]);
            tmax[qi] = t * a.scale_log2;  // the scale is positive
        }
    };
    // Lazy rescale: the reference max moves only when some row's max has
    // grown by more than kRescale (log2 units), so O and l stay in registers
    // untouched on most tiles.  Exact: O and l are both taken relative to
    // the same reference, and probabilities stay below 2^kRescale.  Some
    // row has grown that much iff some lane's own maximum has, so the
    // cross-lane reduction runs only on the tiles that rescale.
    auto rescale = [&](const auto &tmax) {
        constexpr int NQ = sizeof(tmax) / sizeof(tmax[0]);
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if (__any(tmax[qi] > mrun[qi] + kRescale)) {
                const float mnew = fmaxf(mrun[qi], max_over_kgroups(tmax[qi]));
                const float alpha = fast_exp2(mrun[qi] - mnew);
                mrun[qi] = mnew;
                lpart[qi] *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[qi][db] *= alpha;
            }
        }
    };
    // probabilities against the reference max, their row sums, and P^T as
    // the B operand of the 32-key steps: slots 0-3 hold keys 32*ks + 4*kg +
    // (0..3), slots 4-7 keys 32*ks + 16 + 4*kg + (0..3)
    auto exps = [&](auto &sc, auto &pb) {
        constexpr int NQ = sizeof(sc) / sizeof(sc[0]);
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            const float mref = mrun[qi];
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sc[qi][kb][e] = fast_exp2(fmaf(sc[qi][kb][e], a.scale_log2, -mref));
                    psum += sc[qi][kb][e];
                }
            lpart[qi] += psum;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pb[qi][ks][e] = static_cast<__bf16>(sc[qi][2 * ks][e]);
                    pb[qi][ks][4 + e] = static_cast<__bf16>(sc[qi][2 * ks + 1][e]);
                }
        }
    };
    // O^T += V^T P^T over NKS*NDB steps (ks, db); each V^T fragment (two
    // transpose loads) serves every block and is read kVPre steps ahead;
    // four base pointers per tile (one per swizzle class db & 3), the rest
    // of each address a compile-time constant
    auto pv = [&](uint32_t sbase, const auto &pb) {
        constexpr int NQ = sizeof(pb) / sizeof(pb[0]);
        constexpr int NSTEP = NKS * NDB;
        constexpr int kVPre = 4;
        const lds_u8 *vbase[4];
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4)
            vbase[d4] = reinterpret_cast<const lds_u8 *>(static_cast<uintptr_t>(sbase + voff[d4])) +
                        wk * NKS * 32 * ROWB;
        auto vptr = [&](int n) {
            const int ks = n / NDB, db = n % NDB;
            return vbase[db & 3] + (db >> 2) * 128 + ks * 32 * ROWB;
        };
        bf16x4 vlo[kVPre], vhi[kVPre];
#pragma unroll
        for (int n = 0; n < kVPre; ++n) {
            vlo[n] = lds_read_tr16(vptr(n));
            vhi[n] = lds_read_tr16(vptr(n) + 16 * ROWB);
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
                vlo[n % kVPre] = lds_read_tr16(vptr(n + kVPre));
                vhi[n % kVPre] = lds_read_tr16(vptr(n + kVPre) + 16 * ROWB);
            }
            const int ks = n / NDB, db = n % NDB;
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) o[qi][db] = mfma16x16x32(vf, pb[qi][ks], o[qi][db]);
        }
    };

    // One pass over this key group's part of tile i for query blocks
    // 0 .. NQ-1.  KIND is the tile's kind, known before the call: a full
    // cache tile (no masking) or a masked one -- a partial cache tile (keys
    // past the split's end) or a packed tile (tree mask).  A separate
    // instance keeps the common full-tile path free of the masking code and
    // of the register copies that merging the paths would need.
    auto compute_tile = [&](int i, uint32_t sbase, auto nq_c, auto kind_c) {
        constexpr int NQ = decltype(nq_c)::value;
        constexpr int KIND = decltype(kind_c)::value;
        const int wi = 2 * (i - ncache);
        const bool packed = KIND == kTileMasked && i >= ncache;  // wave-uniform
        uint32_t mw[NQ][2];  // this lane's row's mask words for the tile's two 32-key halves
        if (packed) {
            // A packed tile whose keys are invisible to every row of this
            // wavefront's blocks changes no row's softmax state: skip it.
            // Only ancestors are visible, so with a deep, narrow tree most
            // packed tiles are invisible to a given block of 16 rows.
            bool any = false;
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                // the second word exists unless the tile is the last and P_max <= 32*(2*tile+1);
                // it is read from a clamped index and then dropped (a select of loaded
                // values, not of addresses, which would put the operands in scratch)
                const uint32_t w1 = mwords[lt[qi] * a.nw + min(wi + 1, a.nw - 1)];
                mw[qi][0] = mwords[lt[qi] * a.nw + wi];
                mw[qi][1] = (wi + 1 < a.nw) ? w1 : 0u;
                any |= (KSPLIT == 2 ? (wk == 0 ? mw[qi][0] : mw[qi][1]) : (mw[qi][0] | mw[qi][1])) != 0u;
            }
            if (!__any(any)) return;
        }
        f32x4 sc[NQ][NKB];
        qk_scores(sbase, sc);

        // mask (partial cache tiles and packed tiles only), online softmax;
        // key of sc[qi][kb][e] within the tile is (wk*NKB + kb)*16 + 4*kg + e
        // cache key j of the tile is valid iff pos(j) < nck; packed key j
        // iff j < lim and its mask bit is set
        if (KIND == kTileMasked && !packed) {
            const int ic = tile_ic(i);
            const int lim = nck;
            // partial cache tile: key j is valid iff its position is below lim
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = (wk * NKB + kb) * 16 + 4 * kg + e;
                        sc[qi][kb][e] = (ic * kblk + kmul * j < lim) ? sc[qi][kb][e] : -INFINITY;
                    }
        } else if (packed) {
            const int lim = tok_hi - (i - ncache) * kBlockN;
            // packed tile: key j = jj + 4*kg (jj = (wk*NKB + kb)*16 + e) is
            // visible iff j < lim and bit j of the row's mask words is set.
            // j stays in jj's 16-key block, so its word is chosen by jj and its
            // bit is bit (jj & 31) of the word shifted right by 4*kg once.
            const int lim2 = lim - 4 * kg;
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                const uint32_t s0 = mw[qi][0] >> (4 * kg), s1 = mw[qi][1] >> (4 * kg);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const int jb = (wk * NKB + kb) * 16;  // wave-uniform
                    const uint32_t sw = (jb < 32) ? s0 : s1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int jj = jb + e;
                        const bool vis = (jj < lim2) && ((sw >> ((kb * 16 + e) & 31)) & 1u);
                        sc[qi][kb][e] = vis ? sc[qi][kb][e] : -INFINITY;
                    }
                }
            }
        }
        float tmax[NQ];
        tile_max(sc, tmax);
        rescale(tmax);
        bf16x8 pb[NQ][NKS];
        exps(sc, pb);
        pv(sbase, pb);
    };
    // Ring of NS LDS stages.  Tiles 0..NS-2 are issued up front.
    // At the top of tile i this wavefront's loads of tile i have landed once
    // at most (NS-2)*2*NLD of its loads remain outstanding; the barrier
    // publishes every wavefront's share and certifies that all reads of the
    // slot of tile i-1 are done, so tile i+NS-1 may be loaded into it.
    // Tiles past the last still issue their loads, all out of range, so
    // every wait counts the same number of loads.
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue_tile(st, st);
    // this lane's query rows (row_of).  Valid blocks form a prefix in qi; a
    // wavefront multiplies only its valid ones (none: it only helps with the
    // loads).
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
        nact += (row0 + row_of(qi, 0) < Mb) ? 1 : 0;
        const int r = row0 + row_of(qi, lq);
        const bool rvalid = r < Mb;
        const int p = rvalid ? r / a.G : 0;
        const int h = g * a.G + (rvalid ? r % a.G : 0);
        lt[qi] = rvalid ? p - tok_lo : 0;
        const uint16_t *qrow = a.q + ((static_cast<size_t>(b) * a.P + p) * a.Hq + h) * D;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
            qf[qi][kc] = as_bf16x8(rvalid ? ld16(qrow + 32 * kc + 8 * kg) : make_uint4(0, 0, 0, 0));
    }
    nact = __builtin_amdgcn_readfirstlane(nact);
    // tokens of this block and their tree-mask rows, staged in LDS once
    if (npk > 0) {
        const int ntok = tok_hi - tok_lo;
        const uint32_t *msrc = a.mask + (static_cast<size_t>(b) * a.P + tok_lo) * a.nw;
        for (int i = tid; i < ntok * a.nw; i += NT) mwords[i] = msrc[i];
    }
    // The Q and mask loads are issued after the ring's first tiles, so
    // their latency overlaps that of the ring; at a first use inside the
    // loop the compiler would wait for them (and for all earlier loads), so
    // they are made to land here, where that wait costs nothing extra.
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi)
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) asm volatile("" : "+v"(qf[qi][kc]));

    // Two runs of the same ring loop: the full cache tiles, then the masked
    // ones.  Separate loops keep the two compute instances' temporaries out
    // of each other's way (one loop holding both measured register spills).
    // Tile i sits in ring slot i % NS; tile i + NS - 1 is loaded into the
    // slot of tile i - 1.
    const int nact_u = nact;
    // calls f(integral_constant<NQ>) with NQ = the wavefront's valid blocks (nothing for none)
    auto with_nq = [&](auto f) {
        if (QPW == 2 && nact_u == 2) f(std::integral_constant<int, QPW>{});
        else if (nact_u >= 1) f(std::integral_constant<int, 1>{});
    };
    auto tile_step = [&](int i, auto kind_c) {
        vm_wait<(NS - 2) * 2 * NLD>();
        __syncthreads();
        const int cslot = i % NS;
        issue_tile(i + NS - 1, (cslot + NS - 1) % NS);
        const uint32_t sbase = lds0 + cslot * STAGEB;
        with_nq([&](auto nq_c) { compute_tile(i, sbase, nq_c, kind_c); });
    };
    for (int i = 0; i < nfull; ++i) tile_step(i, std::integral_constant<int, kTileFull>{});
    for (int i = nfull; i < ntile; ++i) tile_step(i, std::integral_constant<int, kTileMasked>{});
    vm_wait<0>();

    // per-row sums over the four k-groups of the lane's column
    float lsum[QPW];
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
        lsum[qi] = lpart[qi] + shfl_xor(lpart[qi], 16);
        lsum[qi] += shfl_xor(lsum[qi], 32);
    }
    if (KSPLIT == 2) {
        // key group 1 hands (m, l, O) to key group 0 through LDS (the ring is
        // drained), which merges: M = max(m0, m1), O = O0 2^(m0-M) + O1 2^(m1-M)
        __syncthreads();
        float *xo = reinterpret_cast<float *>(stage);                  // [NQG][QPW][NDB][64] f32x4
        float *xm = xo + NQG * QPW * NDB * 64 * 4;                      // [NQG][QPW][64] m, l
        if (wk == 1) {
#pragma unroll
            for (int qi = 0; qi < QPW; ++qi) {
                if (qi >= nact) break;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    *reinterpret_cast<f32x4 *>(xo + (((wq * QPW + qi) * NDB + db) * 64 + lane) * 4) = o[qi][db];
                xm[((wq * QPW + qi) * 64 + lane) * 2] = mrun[qi];
                xm[((wq * QPW + qi) * 64 + lane) * 2 + 1] = lsum[qi];
            }
        }
        __syncthreads();
        if (wk == 1) return;
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) {
            if (qi >= nact) break;
            const float m1 = xm[((wq * QPW + qi) * 64 + lane) * 2];
            const float l1 = xm[((wq * QPW + qi) * 64 + lane) * 2 + 1];
            const float M = fmaxf(mrun[qi], m1);
            const float a0 = fast_exp2(mrun[qi] - M), a1 = fast_exp2(m1 - M);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const f32x4 o1 = *reinterpret_cast<const f32x4 *>(xo + (((wq * QPW + qi) * NDB + db) * 64 + lane) * 4);
                o[qi][db] = o[qi][db] * a0 + o1 * a1;
            }
            mrun[qi] = M;
            lsum[qi] = lsum[qi] * a0 + l1 * a1;
        }
    }

#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
        const int r = row0 + row_of(qi, lq);
        const bool rvalid = r < Mb;
        if (a.nsplit == 1) {
            // o[qi][db][e] = O[query r][d = db*16 + 4*kg + e]; padding rows get zeros
            if (r < Mpad) {
                const float inv = (rvalid && lsum[qi] > 0.f) ? 1.f / lsum[qi] : 0.f;
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
            if (kg == 0) a.ws_ml[prow] = make_float2(mrun[qi], lsum[qi]);
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
template <int D, bool PAGED>
__global__ __launch_bounds__(64) void k_tree_attn_f32(const float *__restrict__ q, const float *__restrict__ k_new,
                                                      const float *__restrict__ v_new,
                                                      const float *__restrict__ k_cache,
                                                      const float *__restrict__ v_cache,
                                                      const int32_t *__restrict__ kv_len,
                                                      const uint32_t *__restrict__ mask,
                                                      const int32_t *__restrict__ plen, int P, int Hq,
                                                      int Hkv, int S_max, int nw, float scale_log2,
                                                      float *__restrict__ out, AttnArgs pg) {
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
            size_t row;
            if constexpr (PAGED) {
                const int64_t page = min(max(static_cast<int64_t>(pg.bt[static_cast<size_t>(b) * pg.max_pages +
                                                                       j / pg.page_size]),
                                             static_cast<int64_t>(0)),
                                         pg.num_pages - 1);
                row = (static_cast<size_t>(page) * Hkv + g) * pg.page_size + j % pg.page_size;
            } else {
                row = (static_cast<size_t>(b) * Hkv + g) * S_max + j;
            }
            kr = k_cache + row * D;
            vr = v_cache + row * D;
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

}  // namespace

AttnPlan plan_attention(int dtype, int B, int P_max, int Hq, int Hkv, int D, int S_max) {
    AttnPlan plan{0, 1, kBlockN, 0, 1, 0, 4, 1};
    if (dtype != 1) return plan;  // fp32 path needs no workspace
    const int G = Hq / Hkv;
    const int rows = G * P_max;
    // 16-row query blocks per wavefront: enough that one workgroup holds all
    // rows of a (request, KV head) whenever they fit in 256
    // (QPW, wavefronts, key groups): up to 64 rows (2, 4, 2) -- two
    // query groups, each tile's keys split over two wavefronts, so all four
    // SIMDs work even for a handful of rows; up to 128 rows (2, 4, 1);
    // more (2, 8, 1) = 256 rows per workgroup
    plan.qpw = 2;
    plan.nwave = rows <= 128 ? 4 : 8;
    plan.ksplit = rows <= 64 ? 2 : 1;
    if (rows <= 64 && knob(RD_KNOB_ATTN_FEWROW) != 2) {
        // (1, 8, 2) with lane-interleaved rows: four query groups of ~rows/4
        plan.qpw = 1;
        plan.nwave = 8;
    }
    const int rb = 16 * plan.qpw * plan.nwave / plan.ksplit;
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
    if (knob(RD_KNOB_ATTN_SPLITS) > 0) nsplit = knob(RD_KNOB_ATTN_SPLITS);
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
                            void *ws, hipStream_t stream, const PagedKV *paged) {
    const float sc = (scale == 0.f) ? 1.f / sqrtf(static_cast<float>(D)) : scale;
    const int nw = (P_max + 31) / 32;
    AttnArgs a{};
    if (paged) {
        a.bt = paged->block_table;
        a.max_pages = paged->max_pages;
        a.page_size = paged->page_size;
        a.num_pages = paged->num_pages;
    }
    if (dtype == 0) {
        const dim3 grid(static_cast<unsigned>(static_cast<size_t>(B) * P_max * Hq));
        auto kern = paged ? ((D == 64) ? k_tree_attn_f32<64, true> : k_tree_attn_f32<128, true>)
                          : ((D == 64) ? k_tree_attn_f32<64, false> : k_tree_attn_f32<128, false>);
        hipLaunchKernelGGL(kern, grid, dim3(kWave), 0, stream, static_cast<const float *>(q),
                           static_cast<const float *>(k_new), static_cast<const float *>(v_new),
                           static_cast<const float *>(k_cache), static_cast<const float *>(v_cache), kv_len,
                           mask, plen, P_max, Hq, Hkv, S_max, nw, sc * kLog2e, static_cast<float *>(out), a);
        return hipGetLastError();
    }
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
    // ring depth: three stages (measured on MI355X: two starve the MFMA-heavy
    // shapes, four did not stream faster)
    auto go = [&](auto d_c, auto pg_c) {
        constexpr int DD = decltype(d_c)::value;
        constexpr bool PG = decltype(pg_c)::value;
        if (plan.ksplit == 2 && plan.qpw == 1)
            hipLaunchKernelGGL((k_tree_attn_bf16<DD, 1, 8, 2, 3, true, PG>), grid, blk, 0, stream, a);
        else if (plan.ksplit == 2)
            hipLaunchKernelGGL((k_tree_attn_bf16<DD, 2, 4, 2, 3, false, PG>), grid, blk, 0, stream, a);
        else if (plan.nwave == 4)
            hipLaunchKernelGGL((k_tree_attn_bf16<DD, 2, 4, 1, 3, false, PG>), grid, blk, 0, stream, a);
        else
            hipLaunchKernelGGL((k_tree_attn_bf16<DD, 2, 8, 1, 3, false, PG>), grid, blk, 0, stream, a);
    };
    auto go_d = [&](auto pg_c) {
        if (D == 64)
            go(std::integral_constant<int, 64>{}, pg_c);
        else
            go(std::integral_constant<int, 128>{}, pg_c);
    };
    if (paged)
        go_d(std::true_type{});
    else
        go_d(std::false_type{});
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
