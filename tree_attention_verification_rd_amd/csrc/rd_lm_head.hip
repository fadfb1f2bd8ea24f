// Step 3: output projection and greedy target token.
//
// Greedy verification (Apple/NVIDIA ReDrafter news article, greedy-decoding
// benchmark paragraph) needs the target's argmax over the vocabulary at
// every packed position: logits = hidden . W^T, argmax taken on the fp32
// accumulators with the lowest vocabulary id winning ties.
//
// bf16 GEMM layout.  Only valid packed rows (p < packed_len[b]) are
// computed: every workgroup numbers them itself with a prefix sum over the
// packed lengths (no separate pass, no launch).  The product is
// formed transposed, C^T = W X^T (A operand = weight rows, B operand =
// hidden rows), so each lane's accumulator holds four consecutive
// vocabulary entries of one row -- what the argmax epilogue and the logits
// store want.  Both operands are staged through LDS by direct global->LDS
// loads (no registers, whole cache lines per instruction) into a ring of
// k-steps, and each multiplying wavefront computes a WV x WR block out of
// LDS with v_mfma_f32_16x16x32_bf16: in the few-row shape four such
// wavefronts plus four that only issue the loads, in the many-row shape
// eight that both load and multiply.  The epilogue reduces
// (max, first index) over the tile's vocabulary range and writes one
// partial per (row, vocabulary tile); a second kernel reduces the partials
// in a fixed order.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "../../include/rd.h"
#include "rd_common.h"
#include "rd_internal.h"

namespace rd {

namespace {

// Fixed device scratch of rd_lm_head_argmax_noalloc: the per-(row,
// vocabulary tile) argmax partials live here instead of in a caller's
// workspace.  Every device the library runs on holds its own copy for the
// life of the process; calls on one device share it.
static __device__ __align__(256) uint8_t scratch[RD_NOALLOC_SCRATCH_BYTES];


struct LmArgs {
    const uint16_t *hidden, *weight;
    const int32_t *plen;  // packed lengths [B] (clamped to [0, P]); null: all P rows valid
    int B, P, K, V;
    uint16_t *logits;
    // null: logits row b*P + p is packed row b*P + p; otherwise logits is the
    // unpacked [B, W, L, V] output and the row goes to output row
    // node_row[b*P + p] (the node's first candidate; the unpack gather
    // folded into the epilogue)
    const int32_t *node_row;
    float *pval;
    int32_t *pidx;
    int nvt, nrt;
};

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// Block-wide inclusive prefix sum of one value per thread (NT threads);
// `tot` receives the sum.  `scratch` holds NT/64 ints.
template <int NT>
__device__ __forceinline__ int block_scan(int v, int *scratch, int &tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off, kWave);
        if (lane >= off) v += t;
    }
    if (lane == 63) scratch[wave] = v;
    __syncthreads();
    int before = 0;
    tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int sw = scratch[w];
        before += (w < wave) ? sw : 0;
        tot += sw;
    }
    __syncthreads();
    return v + before;
}

// Block-wide inclusive prefix maximum of one value per thread (NT threads).
template <int NT>
__device__ __forceinline__ int block_scan_max(int v, int *scratch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off, kWave);
        if (lane >= off) v = max(v, t);
    }
    if (lane == 63) scratch[wave] = v;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) v = (w < wave) ? max(v, scratch[w]) : v;
    __syncthreads();
    return v;
}

// Valid rows (p < packed_len[b]) are numbered in (b, p) order -- the compact
// rows.  count_rows returns their number; with B <= NT thread b also keeps
// its request's first compact row and row count (st, cnt), so that
// map_rows need not read the lengths again.
template <int NT>
__device__ int count_rows(const int32_t *plen, int B, int P, int *scratch, int &st, int &cnt) {
    int carry = 0;
    st = 0;
    cnt = 0;
    for (int b0 = 0; b0 < B; b0 += NT) {
        const int b = b0 + static_cast<int>(threadIdx.x);
        const int n = (b < B) ? (plen ? min(max(plen[b], 0), P) : P) : 0;
        int tot;
        const int incl = block_scan<NT>(n, scratch, tot);
        if (b0 == 0) {
            st = incl - n;
            cnt = n;
        }
        carry += tot;
    }
    return carry;
}
// rmap[t] = packed row b*P + p of compact row r0 + t, t < n <= BR.  Each
// request whose rows meet the range marks the tile row where they begin;
// a prefix maximum over the tile rows then gives every row its request.
template <int NT, int BR>
__device__ void map_rows(const int32_t *plen, int B, int P, int r0, int n, int st, int cnt, int32_t *rmap,
                         int32_t *head, int32_t *hstart, int *scratch) {
    const int tid = static_cast<int>(threadIdx.x);
    for (int i = tid; i < BR; i += NT) head[i] = -1;
    __syncthreads();
    auto mark = [&](int b, int s0, int c) {
        if (c > 0 && s0 < r0 + n && s0 + c > r0) {
            const int pos = max(s0, r0) - r0;  // distinct for distinct non-empty requests
            head[pos] = b;
            hstart[pos] = s0;
        }
    };
    if (B <= NT) {
        if (tid < B) mark(tid, st, cnt);
    } else {
        int carry = 0;
        for (int b0 = 0; b0 < B; b0 += NT) {
            const int b = b0 + tid;
            const int c = (b < B) ? (plen ? min(max(plen[b], 0), P) : P) : 0;
            int tot;
            const int s0 = carry + block_scan<NT>(c, scratch, tot) - c;
            if (b < B) mark(b, s0, c);
            carry += tot;
        }
    }
    __syncthreads();
    // tile row 0 always holds a mark (the request containing row r0)
    const int at = block_scan_max<NT>((tid < BR && tid < n && head[tid] >= 0) ? tid : -1, scratch);
    if (tid < n && tid < BR) rmap[tid] = head[at] * P + (r0 + tid - hstart[at]);
}

// SPEC: eight wavefronts, two per SIMD -- wavefronts 0-3 only multiply,
// wavefronts 4-7 only issue the ring loads.  A load stalled at issue (the
// memory pipeline full) then holds up only its own wavefront, while the
// SIMD's multiplying wavefront keeps the MFMA pipe fed.  Needs a wave tile
// that fits 256 registers.
// NWV: wavefronts that both load and multiply (4, or 8 for two per SIMD;
// with SPEC four of each kind).
template <int WV, int WR, int GV, int GR, int NSW, int NSX, int BK, bool KROT, bool SPEC, int NWV = 4>
__global__ __launch_bounds__(SPEC ? 512 : 64 * NWV, 1) void k_lm_head_bf16(LmArgs a) {
    constexpr int NCW = SPEC ? 4 : NWV;  // multiplying wavefronts
    constexpr int NLD = SPEC ? 4 : NWV;  // loading wavefronts
    constexpr int NT = SPEC ? 512 : 64 * NWV;
    static_assert(GV * GR == NCW, "one wave tile per multiplying wavefront");
    static_assert(NSX >= 2 && NSW >= NSX, "each ring needs a stage in flight while another is consumed");
    static_assert(BK == 32 || BK == 64, "one or two 32-wide MFMA steps per k-step");
    constexpr int NSUB = BK / 32;            // MFMA k-steps per staged k-step
    constexpr int BV = GV * WV;              // vocabulary rows per tile
    constexpr int BR = GR * WR;              // compact hidden rows per tile
    constexpr int NVB = WV / 16;
    constexpr int NRB = WR / 16;
    constexpr int kRowB = BK * 2;            // bytes of one staged row (a cache line or half of one)
    constexpr int CPR = BK / 8;              // 16-byte chunks per staged row
    constexpr int RPL = 1024 / kRowB;        // rows per 1 KB load instruction
    constexpr int kWStage = BV * kRowB;      // bytes of one weight stage
    constexpr int kXStage = BR * kRowB;      // bytes of one hidden stage
    constexpr int kXBase = NSW * kWStage;    // hidden ring after the weight ring
    constexpr int NL = (BV + BR) / RPL / NLD;  // LDS loads per loading wavefront per k-step (both operands)
    constexpr int NLW = BV / RPL / NLD;        // ... of weight rows
    constexpr int NLX = BR / RPL / NLD;        // ... of hidden rows
    static_assert(BV % (NLD * RPL) == 0 && BR % (NLD * RPL) == 0, "each wavefront loads whole groups of both operands");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NSW * kWStage + NSX * kXStage];
    __shared__ int32_t rmap[BR];  // packed row (b*P + p) of each compact row of the tile
    __shared__ int32_t rhead[BR], rhstart[BR];
    __shared__ int scan_tmp[NT / 64];

    // wave-uniform values are read into scalar registers explicitly so the
    // buffer resources built from them stay scalar (no per-lane loops)
    int my_st, my_cnt;
    const int R = __builtin_amdgcn_readfirstlane(count_rows<NT>(a.plen, a.B, a.P, scan_tmp, my_st, my_cnt));
    const int nrt = (R + BR - 1) / BR;       // row tiles that hold valid rows
    const int ntiles = nrt * a.nvt;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 15;
    const int kg = lane >> 4;
    const bool loader = SPEC && wave >= 4;   // issues loads only
    const bool issues = !SPEC || loader;     // issues ring loads
    const int cw = SPEC ? (wave & 3) : wave;  // index among the multiplying wavefronts
    const int lw = SPEC ? (wave & 3) : wave;  // index among the loading wavefronts
    const int gv = cw % GV;
    const int gr = cw / GV;
    const int K = a.K;
    const int nk = (K + BK - 1) / BK;
    const uint32_t rowb = static_cast<uint32_t>(K) * 2;

    // Staging.  A stage holds BV weight rows then BR hidden rows, BK
    // columns each (128 or 64 bytes per row).  Each load instruction moves
    // RPL whole rows; within a row the 16-byte chunks are stored XOR-swizzled
    // (by row & 7 for 8 chunks, by (row >> 1) & 3 for 4), so the fragment
    // reads below (16 rows x one chunk per instruction) hit distinct banks.
    // Lane i of a load covers staged row RPL*j + i/CPR and stores LDS slot
    // i % CPR, which holds chunk slot ^ swizzle(row).  Load j = NLD*i + lw
    // (lw: the index among the NLD loading wavefronts) is that wavefront's
    // i-th: its first NLW loads are weight rows, the rest hidden rows.
    auto swz = [](int row) { return CPR == 8 ? (row & 7) : ((row >> 1) & 3); };
    const int lrow = lane / CPR;
    const int lchunk = (lane % CPR) ^ swz(lrow);
    const i32x4_t xres = make_srsrc(a.hidden, static_cast<uint32_t>(static_cast<size_t>(a.B) * a.P * K * 2));
    const uint32_t lds0 = lds_addr_of(lds);
    // fragment reads: lane reads row lq of each 16-row block, k-chunk
    // 4*ks + kg, at its swizzled slot; the ks = 1 slot is the ks = 0 slot
    // with chunk bit 2 flipped
    const uint32_t sw = static_cast<uint32_t>((kg ^ swz(lq)) << 4);
    const uint32_t aoff = static_cast<uint32_t>(gv * WV + lq) * kRowB + sw;
    const uint32_t boff = static_cast<uint32_t>(gr * WR + lq) * kRowB + sw;
    // All workgroups on one XCD (block i runs on XCD i % 8) walk K in the
    // same order and mostly run side by side, so the rows they share are
    // fetched into that XCD's L2 once.  With KROT the XCDs start at
    // different k-steps, so that they do not all address the same offset of
    // the power-of-two-strided rows at once (which would crowd a few HBM
    // channels).  Both launched shapes use it; a shape without it stays
    // available for measurement.
    const int krot = KROT ? ((blockIdx.x & 7) * nk / 8) % nk : 0;

    // The grid is sized on the host for the largest possible row count, but
    // only tiles with valid rows do work.  The first ntiles workgroups take
    // them, XCD by XCD in contiguous ranges of the tile order (groups of up
    // to GM row tiles walk the vocabulary together); the rest exit.  Since
    // workgroups are dispatched in id order, the idle ones come last instead
    // of interleaving with real ones (which would leave some shader engines
    // with twice the work of others).
    if (static_cast<int>(blockIdx.x) >= ntiles) return;
    constexpr int GM = 8;
    {
        const int t = xcd_tile(blockIdx.x, ntiles);
        const int grp = t / (GM * a.nvt);
        const int gsz = min(GM, nrt - grp * GM);
        const int within = t - grp * GM * a.nvt;
        const int rt = grp * GM + within % gsz;
        const int vt = within / gsz;
        const int r0 = rt * BR;
        const int v0 = vt * BV;
        const int wrows = max(0, min(a.V - v0, BV));
        const i32x4_t wres = make_srsrc(a.weight + static_cast<size_t>(min(v0, a.V)) * K,
                                        static_cast<uint32_t>(wrows) * rowb);
        // weight rows past V fall outside wres; hidden rows past R get kOOB
        const uint32_t wbase = static_cast<uint32_t>(RPL * lw + lrow) * rowb + 16 * lchunk;
        // The weight rows of k-step kt (k-step (kt + krot) mod nk) go to
        // weight-ring slot kt % NSW, its hidden rows to hidden-ring slot
        // kt % NSX.  The weight stream comes from HBM and is issued NSW-1
        // k-steps ahead; the hidden rows are L2 hits and need less lead.
        // Stages past the last k-step still issue their loads, all out of
        // range (zeros), so every wait below counts the same number of loads.
        auto kstep_of = [&](int kt) { return (kt < nk) ? ((kt + krot >= nk) ? kt + krot - nk : kt + krot) : -1; };
        auto issue_w = [&](int kt, int slot) {
            const int kr = kstep_of(kt);
            const bool kin = kr >= 0 && kr * BK + 8 * lchunk < K;
            const uint32_t kadd = static_cast<uint32_t>(kr) * kRowB;
            const uint32_t sbase = lds0 + slot * kWStage + lw * 1024;
#pragma unroll
            for (int i = 0; i < NLW; ++i)
                lds_dma16(sbase + i * NLD * 1024, wres, kin ? wbase + i * NLD * RPL * rowb + kadd : kOOB);
        };
        // The ring's first weight stages depend on the tile alone: they go
        // out before the hidden rows are numbered, so that work overlaps
        // their latency (the issue order of the ring is unchanged).
        if (issues) {
#pragma unroll
            for (int st = 0; st <= NSW - NSX; ++st) issue_w(st, st);
        }
        map_rows<NT, BR>(a.plen, a.B, a.P, r0, min(BR, R - r0), my_st, my_cnt, rmap, rhead, rhstart, scan_tmp);
        __syncthreads();
        uint32_t xbase[NLX];
#pragma unroll
        for (int i = 0; i < NLX; ++i) {
            const int m = r0 + RPL * (NLD * i + lw) + lrow;
            xbase[i] = (m < R) ? static_cast<uint32_t>(rmap[m - r0]) * rowb + 16 * lchunk : kOOB;
        }
        auto issue_x = [&](int kt, int slot) {
            const int kr = kstep_of(kt);
            const bool kin = kr >= 0 && kr * BK + 8 * lchunk < K;
            const uint32_t kadd = static_cast<uint32_t>(kr) * kRowB;
            const uint32_t sbase = lds0 + kXBase + slot * kXStage + lw * 1024;
#pragma unroll
            for (int i = 0; i < NLX; ++i)
                lds_dma16(sbase + i * NLD * 1024, xres, kin ? xbase[i] + kadd : kOOB);
        };
        // a wavefront whose rows are all padding only helps with the loads
        const bool active = !loader && r0 + gr * WR < R;

        f32x4 acc[NVB][NRB];
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) acc[vb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

        // Two LDS rings.  Issue order is: weight stages 0..NSW-NSX-1 alone,
        // then pairs (weight stage j + NSW - NSX, hidden stage j) for j = 0,
        // 1, ...; k-step kt issues the pair with j = kt + NSX - 1.  At the top
        // of k-step kt this wavefront's hidden loads of stage kt -- and so,
        // loads completing in order, its earlier weight loads of stage kt --
        // have landed once at most (NSX-2) pairs remain outstanding; the
        // barrier then publishes every wavefront's share and certifies that
        // all reads of the slots of k-step kt-1 are done, so they may be
        // reloaded.
        //
        // Fragments are software-pipelined across the barrier: the last
        // 32-wide MFMA step of k-step kt is read into registers before the
        // barrier of k-step kt+1 and multiplied after it, so LDS latency does
        // not stall the MFMAs.  (The first k-step multiplies zero fragments in
        // that slot.)  With one MFMA step per k-step the two fragment buffers
        // alternate between k-steps.
        //
        // Within a k-step the multiplies run in chunks, and the ring loads and
        // fragment reads are spread between the chunks.  Issued as one burst
        // after the barrier, they kept the single wavefront of each SIMD from
        // issuing MFMAs until the burst had been accepted: per-k-step stamps
        // showed the loads costing 400-500 cycles on top of ~1200 cycles of
        // multiplies.
        auto mma = [&](const bf16x8 (&fa)[NVB], const bf16x8 (&fb)[NRB]) {
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) acc[vb][rb] = mfma16x16x32(fa[vb], fb[rb], acc[vb][rb]);
        };
        bf16x8 fa2[2][NVB], fb2[2][NRB];  // [1]: the held (previous) step
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) fa2[1][vb] = bf16x8{};
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) fb2[1][rb] = bf16x8{};

        if (issues) {
#pragma unroll
            for (int j = 0; j < NSX - 1; ++j) {
                if (j > 0) issue_w(j + NSW - NSX, j + NSW - NSX);
                issue_x(j, j);
            }
        }

        // The k loop is unrolled by two (the fragment buffers alternate);
        // ring slots are tracked at run time.
        int wslot = 0, xslot = 0;  // slots of k-step kt
        auto step = [&](int kt, auto cur_c) {
            constexpr int cur = decltype(cur_c)::value;  // fragment buffer of this k-step
            vm_wait<(NSX - 2) * NL>();
            __syncthreads();
            // this k-step's loads: weight stage kt+NSW-1, hidden stage kt+NSX-1
            const int krw = kstep_of(kt + NSW - 1), krx = kstep_of(kt + NSX - 1);
            const bool kinw = krw >= 0 && krw * BK + 8 * lchunk < K;
            const bool kinx = krx >= 0 && krx * BK + 8 * lchunk < K;
            const uint32_t kaddw = static_cast<uint32_t>(krw) * kRowB, kaddx = static_cast<uint32_t>(krx) * kRowB;
            const int wsl = (wslot == 0) ? NSW - 1 : wslot - 1, xsl = (xslot == 0) ? NSX - 1 : xslot - 1;
            const uint32_t sbw = lds0 + wsl * kWStage + lw * 1024;
            const uint32_t sbx = lds0 + kXBase + xsl * kXStage + lw * 1024;
            auto issue_one = [&](int j) {
                if (j < NLW)
                    lds_dma16(sbw + j * NLD * 1024, wres, kinw ? wbase + j * NLD * RPL * rowb + kaddw : kOOB);
                else
                    lds_dma16(sbx + (j - NLW) * NLD * 1024, xres, kinx ? xbase[j - NLW] + kaddx : kOOB);
            };
            if (active) {
                const uint8_t *wst = lds + wslot * kWStage;
                const uint8_t *xst = lds + kXBase + xslot * kXStage;
                // The multiplies run in NSUB*NVB chunks of NRB; the loads and
                // this k-step's fragment reads are spread between the chunks
                // so that the MFMA pipe always has work queued.
                constexpr int NCH = NSUB * NVB;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const int h = c / NVB, vb = c % NVB;
                    if (!SPEC) {
                        // this k-step's ring loads go out in the first half of
                        // the chunks, as early as the MFMA stream allows: with
                        // two stages they must land by the next k-step's wait
                        // (spread over all chunks: dedup sweep 7.5 -> 7.0 ms)
#pragma unroll
                        for (int j = (2 * c < NCH ? c * NL / (NCH / 2) : NL); j < (2 * c < NCH ? (c + 1) * NL / (NCH / 2) : NL);
                             ++j)
                            issue_one(j);
                    }
                    // the fragments this chunk multiplies: NSUB == 1, the held
                    // buffer; NSUB == 2, half 0 the held second half of the
                    // previous k-step, half 1 this k-step's first half
                    const int src = (NSUB == 2) ? (h == 0 ? 1 : 0) : (cur ^ 1);
                    const int dst = (NSUB == 2) ? (h == 0 ? 0 : 1) : cur;
                    const uint32_t x = (NSUB == 2 && h == 1) ? 64u : 0u;
                    fa2[dst][vb] = *reinterpret_cast<const bf16x8 *>(wst + ((aoff ^ x) + vb * 16 * kRowB));
#pragma unroll
                    for (int rb = vb * NRB / NVB; rb < (vb + 1) * NRB / NVB; ++rb)
                        fb2[dst][rb] = *reinterpret_cast<const bf16x8 *>(xst + ((boff ^ x) + rb * 16 * kRowB));
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) acc[vb][rb] = mfma16x16x32(fa2[src][vb], fb2[src][rb], acc[vb][rb]);
                    // keep the chunks in this order: nothing moves across
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else if (issues) {
#pragma unroll
                for (int j = 0; j < NL; ++j) issue_one(j);
            }
            wslot = (wslot + 1 == NSW) ? 0 : wslot + 1;
            xslot = (xslot + 1 == NSX) ? 0 : xslot + 1;
        };
        // An odd k-step count gets one padding step (its loads are out of
        // range, so it multiplies zeros); the held buffer is then always [1].
        for (int kt = 0; kt < nk; kt += 2) {
            step(kt, std::integral_constant<int, 0>{});
            step(kt + 1, std::integral_constant<int, 1>{});
        }
        if (active) mma(fa2[1], fb2[1]);
        vm_wait<0>();
        __syncthreads();  // the padding stages' loads have landed before LDS is reused

        // epilogue: acc[vb][rb][e] = logit(row r0 + gr*WR + rb*16 + lq,
        //                                   vocab v0 + gv*WV + vb*16 + 4*kg + e)
        float *redv = reinterpret_cast<float *>(lds);
        int32_t *redi = reinterpret_cast<int32_t *>(lds + GV * BR * 4);
        // the loading wavefronts hold no results
        if (!loader) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                const int row = gr * WR + rb * 16 + lq;
                const int m = r0 + row;
                const bool mvalid = m < R;
                float bv = -INFINITY;
                int bi = 0x7fffffff;
                if (active) {
                    const int pr = mvalid ? rmap[m - r0] : 0;
                    const int64_t orow = (a.node_row && mvalid) ? a.node_row[pr] : pr;
#pragma unroll
                    for (int vb = 0; vb < NVB; ++vb) {
                        const int v = v0 + gv * WV + vb * 16 + 4 * kg;
                        // candidates come in increasing vocabulary order, so a
                        // strict compare keeps the first of equal values
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const bool take = (v + e < a.V) & (acc[vb][rb][e] > bv);
                            bv = take ? acc[vb][rb][e] : bv;
                            bi = take ? v + e : bi;
                        }
                        if (a.logits && mvalid) {
                            uint16_t *dst = a.logits + static_cast<size_t>(orow) * a.V + v;
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
                    if (GV == 1) {
                        if (mvalid) {
                            const size_t pr = static_cast<size_t>(rmap[m - r0]);
                            a.pval[pr * a.nvt + vt] = bv;
                            a.pidx[pr * a.nvt + vt] = bi;
                        }
                    } else {
                        redv[gv * BR + row] = bv;
                        redi[gv * BR + row] = bi;
                    }
                }
            }
        }
        if (GV > 1) {
            __syncthreads();
            const int rvalid = min(BR, R - r0);
            for (int i = tid; i < rvalid; i += NT) {
                float bv = redv[i];
                int bi = redi[i];
#pragma unroll
                for (int g = 1; g < GV; ++g)
                    if (better(redv[g * BR + i], redi[g * BR + i], bv, bi)) {
                        bv = redv[g * BR + i];
                        bi = redi[g * BR + i];
                    }
                const size_t pr = static_cast<size_t>(rmap[i]);
                a.pval[pr * a.nvt + vt] = bv;
                a.pidx[pr * a.nvt + vt] = bi;
            }
        }
    }
}

// fp32 path: one workgroup per (padded row, 256-wide vocabulary tile)
__global__ __launch_bounds__(256) void k_lm_head_f32(const float *__restrict__ hidden,
                                                     const int32_t *__restrict__ plen,
                                                     const float *__restrict__ weight, int P, int K, int V,
                                                     float *__restrict__ logits,
                                                     const int32_t *__restrict__ node_row,
                                                     float *__restrict__ pval, int32_t *__restrict__ pidx, int nvt) {
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
    if (v < V && logits) logits[(node_row ? static_cast<size_t>(node_row[pr]) : pr) * V + v] = acc;
    rv[threadIdx.x] = (v < V) ? acc : -INFINITY;
    ri[threadIdx.x] = (v < V) ? v : 0x7fffffff;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (static_cast<int>(threadIdx.x) < off &&
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
    // four independent loads per lane per round (index clamped into the row,
    // extras masked), so a row of up to 256 tiles costs one memory round trip
    const float *rv = pval + pr * nvt;
    const int32_t *ri = pidx + pr * nvt;
    for (int i0 = 0; i0 < nvt; i0 += 4 * kWave) {
        float v[4];
        int ix[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = min(i0 + u * kWave + lane, nvt - 1);
            v[u] = rv[i];
            ix[u] = ri[i];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + u * kWave + lane < nvt && better(v[u], ix[u], bv, bi)) {
                bv = v[u];
                bi = ix[u];
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

}  // namespace

// Device address of this device's `scratch`.  The array's name is only a
// host-side stand-in for it, so the address is looked up once per device
// (with that device current) and kept; kernels receive it as an argument.
hipError_t noalloc_scratch(void **out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

LmPlan plan_lm_head(int dtype, int B, int P_max, int K, int V) {
    LmPlan plan{};
    plan.rows_pad = B * P_max;
    if (dtype == 0) {
        plan.vtile = 256;
        plan.rtile = 1;
        plan.variant = 0;
    } else {
        // Two tile shapes.  Few rows (the weight stream dominates): 128
        // vocabulary x 256 rows per tile, 128x64 per multiplying wavefront,
        // k-steps of 64, three weight and three hidden stages -- twice as many
        // tiles to spread over the CUs -- with four more wavefronts that only
        // issue the loads (measured at llama_mha size: 77-80 us against 89-94
        // us with one wavefront per SIMD doing both).  Many rows (the MFMAs
        // dominate): 256 x 256 per tile -- a third less L2 traffic per flop
        // -- over eight wavefronts of 128x64 that all load and multiply, two
        // per SIMD, so one's stalled load issue leaves the MFMA pipe to the
        // other; k-steps of 64 and two stages of each operand (measured
        // against four wavefronts of 128x128 with k-steps of 32 and 5 + 4
        // stages: gqa 1590 vs 1675 us, long_ctx 473 vs 522, dedup_p0.5
        // 6938 vs 7144).  (Ring depths measured on MI355X: deeper weight
        // rings slow the few-row shape.)
        // The RD_KNOB_LM_SHAPE knob forces one.
        const int forced = knob(RD_KNOB_LM_SHAPE);
        plan.variant = forced == 1 ? 0 : forced == 2 ? 1 : (plan.rows_pad > 512 ? 1 : 0);
        plan.vtile = plan.variant ? 256 : 128;
        plan.rtile = 256;
    }
    plan.nvt = (V + plan.vtile - 1) / plan.vtile;
    const size_t rows = static_cast<size_t>(plan.rows_pad);
    plan.ws_bytes = 2 * align256(rows * plan.nvt * 4);
    return plan;
}

hipError_t launch_lm_head(int dtype, const LmPlan &plan, const void *hidden, const int32_t *plen,
                          const void *weight, int B, int P_max, int K, int V, void *logits, int32_t *argmax,
                          void *ws, hipStream_t stream, const int32_t *node_row) {
    char *w = static_cast<char *>(ws);
    const size_t rows = static_cast<size_t>(plan.rows_pad);
    float *pval = reinterpret_cast<float *>(w);
    int32_t *pidx = reinterpret_cast<int32_t *>(w + align256(rows * plan.nvt * 4));

    if (dtype == 0) {
        hipLaunchKernelGGL(k_lm_head_f32, dim3(static_cast<unsigned>(rows * plan.nvt)), dim3(256), 0, stream,
                           static_cast<const float *>(hidden), plen, static_cast<const float *>(weight), P_max, K,
                           V, static_cast<float *>(logits), node_row, pval, pidx, plan.nvt);
    } else {
        LmArgs a;
        a.hidden = static_cast<const uint16_t *>(hidden);
        a.weight = static_cast<const uint16_t *>(weight);
        a.plen = plen;
        a.B = B;
        a.P = P_max;
        a.K = K;
        a.V = V;
        a.logits = static_cast<uint16_t *>(logits);
        a.node_row = node_row;
        a.pval = pval;
        a.pidx = pidx;
        a.nvt = plan.nvt;
        a.nrt = static_cast<int>((rows + plan.rtile - 1) / plan.rtile);
        const dim3 grid(static_cast<unsigned>(a.nrt * a.nvt));
        if (plan.variant == 0)
            hipLaunchKernelGGL((k_lm_head_bf16<128, 64, 1, 4, 3, 3, 64, true, true>), grid, dim3(512), 0, stream, a);
        else
            hipLaunchKernelGGL((k_lm_head_bf16<128, 64, 2, 4, 2, 2, 64, true, false, 8>), grid, dim3(512), 0, stream, a);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_argmax_reduce, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, stream, pval,
                       pidx, plen, B, P_max, plan.nvt, argmax);
    return hipGetLastError();
}

}  // namespace rd
