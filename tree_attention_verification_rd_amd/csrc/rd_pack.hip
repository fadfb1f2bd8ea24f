// Step 1 (pack) and step 1b (tree-causal mask) kernels.
//
// Pack follows dynamic tree attention (Apple/NVIDIA ReDrafter news article,
// "Dynamic tree attention"; ReDrafter paper abstract, point 2): a slot per
// distinct prefix.  Slot order is the first occurrence in a beam-major scan.
//
// One workgroup per request; in every wavefront lane w stands for beam w.
// Depth by depth, the node of (beam w, depth l) is the pair (node at depth
// l-1, token at l); lane w names it by f_l(w), the lowest beam with the same
// pair (w itself when no earlier beam shares the prefix), found by reading
// the other lanes' parent names and tokens with v_readlane.  The NWV
// wavefronts each scan a quarter of the beams and take the minimum of their
// answers through LDS (one barrier per depth), so the scan is W*L/NWV
// iterations of a few branch-free instructions.  A prefix shared with an earlier beam stays
// shared at every shallower depth, so m_w = #{l : f_l(w) < w} is the length
// of the prefix beam w shares with an earlier beam.  Beam w contributes the L - m_w new slots at depths
// m_w..L-1; their positions come from an exclusive prefix sum of those
// counts across lanes, built from five ballots (one per bit of the count)
// and popcounts of the lanes below.  Slot of (w, l) = base(o) + l - m(o)
// with o = f_l(w), read from lane o by a shuffle.
#include "rd_common.h"
#include "rd_internal.h"

namespace rd {

// Packs request b with all NWV wavefronts of the workgroup (every thread
// must call it; it contains workgroup barriers); wavefront 0 writes the
// outputs.  sb and sf are LDS scratch of W*L ints (the beams, the node
// names), fpart of 2*NWV*kWave ints; when su (LDS) is given the unpacker rows
// are also left there for the fused mask.  A ragged request uses only its
// first Wb beams and Lb positions (inflight batching mixes requests of
// different shapes); its padding candidates open no node and get unpacker
// -1.  Returns the packed length (in every lane of wavefront 0).
template <int NWV>
__device__ __forceinline__ int pack_request(const int32_t *__restrict__ beams, int b, int W, int L, int Wb, int Lb,
                                            int32_t *__restrict__ tokens, int32_t *__restrict__ plen,
                                            int32_t *__restrict__ unpacker, int32_t *__restrict__ depth,
                                            int32_t *__restrict__ src, int32_t *sb, int32_t *sf, int32_t *fpart,
                                            int32_t *su) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wq = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int P = W * L;
    const int32_t *bb = beams + static_cast<size_t>(b) * P;
    for (int i = threadIdx.x; i < P; i += NWV * kWave) sb[i] = bb[i];
    __syncthreads();

    const bool active = lane < W;  // writes an unpacker row
    const bool real = lane < Wb;   // a beam of the request
    const int own0 = active ? lane * L : 0;
    // this wavefront's share of the beams to compare against
    const int vchunk = (Wb + NWV - 1) / NWV;
    const int v0 = min(Wb, wq * vchunk), v1 = min(Wb, v0 + vchunk);
    int fprev = 0;  // every beam hangs off the same virtual root
    int m = 0;
    for (int l = 0; l < Lb; ++l) {  // uniform
        const int tok = sb[own0 + l];
        int f = lane;
        for (int v = v0; v < v1; ++v) {  // uniform
            const int pv = __builtin_amdgcn_readlane(fprev, v);
            const int tv = __builtin_amdgcn_readlane(tok, v);
            f = (v < f && pv == fprev && tv == tok) ? v : f;
        }
        // the lowest match over all shares (two buffers by depth parity: a
        // buffer is rewritten two depths later, after every wavefront has
        // passed the next depth's barrier and so finished reading it)
        int32_t *fp = fpart + (l & 1) * NWV * kWave;
        fp[wq * kWave + lane] = f;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NWV; ++q) f = min(f, fp[q * kWave + lane]);
        if (wq == 0 && real) sf[own0 + l] = f;
        m += (f < lane) ? 1 : 0;
        fprev = f;
    }
    if (wq != 0) return 0;

    // exclusive prefix sum of new-slot counts over lanes, bit plane by bit plane
    const int cnt = real ? (Lb - m) : 0;  // 0..16: five bits
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    int base = 0, total = 0;
#pragma unroll
    for (int bit = 0; bit < 5; ++bit) {
        const uint64_t bal = __ballot((cnt >> bit) & 1);
        base += __popcll(bal & below) << bit;
        total += __popcll(bal) << bit;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    int32_t *urow = unpacker + static_cast<size_t>(b) * P + own0;
    const size_t row = static_cast<size_t>(b) * P;
    for (int l = 0; l < L; ++l) {  // uniform: every lane takes part in the shuffles
        const bool cand = real && l < Lb;
        const int o = cand ? sf[own0 + l] : 0;
        const int slot = cand ? __shfl(base, o, kWave) + l - __shfl(m, o, kWave) : -1;
        if (active) {
            urow[l] = slot;
            if (su) su[own0 + l] = slot;
            if (cand && l >= m) {  // a node this beam opens
                tokens[row + slot] = sb[own0 + l];
                if (depth) depth[row + slot] = l;
                if (src) src[row + slot] = own0 + l;
            }
        }
    }
    for (int s = total + lane; s < P; s += kWave) {
        tokens[row + s] = -1;
        if (depth) depth[row + s] = -1;
        if (src) src[row + s] = -1;
    }
    if (lane == 0) plen[b] = total;
    return total;
}

constexpr int kPackWaves = 4;  // wavefronts per request (pack and mask)

__global__ __launch_bounds__(kPackWaves * kWave) void k_pack_beams(const int32_t *__restrict__ beams, int W, int L,
                                                                  int32_t *__restrict__ tokens,
                                                                  int32_t *__restrict__ plen,
                                                                  int32_t *__restrict__ unpacker,
                                                                  int32_t *__restrict__ depth,
                                                                  int32_t *__restrict__ src) {
    __shared__ int32_t sb[kMaxBeams * kMaxBeamLen];
    __shared__ int32_t sf[kMaxBeams * kMaxBeamLen];
    __shared__ int32_t fpart[2 * kPackWaves * kWave];
    pack_request<kPackWaves>(beams, blockIdx.x, W, L, W, L, tokens, plen, unpacker, depth, src, sb, sf, fpart,
                             nullptr);
}

// Step 1b.  [SURV] SpecInfer "Token Tree Verifier": bit q of row p is set iff
// slot q is p or an ancestor of p.  The parent of slot unpacker[w,l] is
// unpacker[w,l-1]; every candidate that maps to a slot names the same
// parent, so concurrent writers store the same value.  Each thread then
// takes whole rows: it walks row p's at most L parent links once, setting
// their bits in an LDS copy of the request's mask rows, which the workgroup
// finally writes out in order.  u is request b's unpacker row block (global
// or LDS), n its packed length; parent is LDS scratch of
// kMaxBeams*kMaxBeamLen ints, rows of P*ceil(P/32) words.
__device__ __forceinline__ void mask_request(const int32_t *u, int n, int b, int W, int L, int32_t *parent,
                                             uint32_t *rows, uint32_t *__restrict__ mask) {
    const int P = W * L;
    const int nw = (P + 31) / 32;
    for (int i = threadIdx.x; i < P; i += blockDim.x) parent[i] = -1;
    for (int i = threadIdx.x; i < P * nw; i += blockDim.x) rows[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < P; i += blockDim.x) {
        const int l = i % L;
        const int p = u[i];
        if (p >= 0 && p < P) parent[p] = (l == 0) ? -1 : u[i - 1];
    }
    __syncthreads();
    n = min(max(n, 0), P);
    for (int p = threadIdx.x; p < n; p += blockDim.x) {
        uint32_t *row = rows + p * nw;  // this thread's row alone
        int cur = p;
        for (int step = 0; step < L && cur >= 0 && cur < P; ++step) {
            if (cur < n) row[cur >> 5] |= 1u << (cur & 31);
            cur = parent[cur];
        }
    }
    __syncthreads();
    uint32_t *out = mask + static_cast<size_t>(b) * P * nw;
    for (int i = threadIdx.x; i < P * nw; i += blockDim.x) out[i] = rows[i];
}

// LDS words for the mask rows of the largest request (128 KB)
constexpr int kMaskRowWords = kMaxBeams * kMaxBeamLen * ((kMaxBeams * kMaxBeamLen + 31) / 32);

__global__ __launch_bounds__(256) void k_tree_mask(const int32_t *__restrict__ unpacker,
                                                   const int32_t *__restrict__ plen, int W, int L,
                                                   uint32_t *__restrict__ mask) {
    __shared__ int32_t parent[kMaxBeams * kMaxBeamLen];
    __shared__ uint32_t mask_rows[kMaskRowWords];
    const int b = blockIdx.x;
    mask_request(unpacker + static_cast<size_t>(b) * W * L, plen[b], b, W, L, parent, mask_rows, mask);
}

// Steps 1 and 1b in one launch: the workgroup packs the request (the first
// wavefront leaving its unpacker in LDS), then builds the mask from it.
// bwid / blen (either may be null: all W beams, all L positions) give a
// ragged request's beam count and length.
__global__ __launch_bounds__(kPackWaves * kWave) void k_pack_mask(const int32_t *__restrict__ beams, int W, int L,
                                                   const int32_t *__restrict__ bwid, const int32_t *__restrict__ blen,
                                                   int32_t *__restrict__ tokens, int32_t *__restrict__ plen,
                                                   int32_t *__restrict__ unpacker, int32_t *__restrict__ depth,
                                                   int32_t *__restrict__ src, uint32_t *__restrict__ mask) {
    __shared__ int32_t sb[kMaxBeams * kMaxBeamLen];
    __shared__ int32_t sf[kMaxBeams * kMaxBeamLen];
    __shared__ int32_t su[kMaxBeams * kMaxBeamLen];
    __shared__ int32_t parent[kMaxBeams * kMaxBeamLen];
    __shared__ int32_t fpart[2 * kPackWaves * kWave];
    __shared__ int32_t n_sh;
    __shared__ uint32_t mask_rows[kMaskRowWords];
    const int b = blockIdx.x;
    const int Wb = bwid ? min(max(__builtin_amdgcn_readfirstlane(bwid[b]), 0), W) : W;
    const int Lb = blen ? min(max(__builtin_amdgcn_readfirstlane(blen[b]), 0), L) : L;
    const int n = pack_request<kPackWaves>(beams, b, W, L, Wb, Lb, tokens, plen, unpacker, depth, src, sb, sf, fpart,
                                           su);
    if (threadIdx.x == 0) n_sh = n;
    __syncthreads();
    mask_request(su, n_sh, b, W, L, parent, mask_rows, mask);
}

hipError_t launch_pack_beams(const int32_t *beams, int B, int W, int L, int32_t *tokens,
                             int32_t *plen, int32_t *unpacker, int32_t *depth, int32_t *src,
                             hipStream_t stream) {
    hipLaunchKernelGGL(k_pack_beams, dim3(B), dim3(kPackWaves * kWave), 0, stream, beams, W, L, tokens, plen,
                       unpacker, depth, src);
    return hipGetLastError();
}

hipError_t launch_pack_mask(const int32_t *beams, const int32_t *bwid, const int32_t *blen, int B, int W, int L,
                            int32_t *tokens, int32_t *plen, int32_t *unpacker, int32_t *depth, int32_t *src,
                            uint32_t *mask, hipStream_t stream) {
    hipLaunchKernelGGL(k_pack_mask, dim3(B), dim3(kPackWaves * kWave), 0, stream, beams, W, L, bwid, blen, tokens,
                       plen, unpacker, depth, src, mask);
    return hipGetLastError();
}

hipError_t launch_tree_mask(const int32_t *unpacker, const int32_t *plen, int B, int W, int L,
                            uint32_t *mask, hipStream_t stream) {
    hipLaunchKernelGGL(k_tree_mask, dim3(B), dim3(256), 0, stream, unpacker, plen, W, L, mask);
    return hipGetLastError();
}

}  // namespace rd
