// Internal launchers shared by the C-ABI layer (rd_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rd {

constexpr int kMaxBeams = 64;
constexpr int kMaxBeamLen = 16;

hipError_t launch_pack_beams(const int32_t *beams, int B, int W, int L, int32_t *tokens,
                             int32_t *plen, int32_t *unpacker, int32_t *depth, int32_t *src,
                             hipStream_t stream);
// bwid / blen: per-request beam count and length of a ragged batch, or null (full W, L)
hipError_t launch_pack_mask(const int32_t *beams, const int32_t *bwid, const int32_t *blen, int B, int W, int L,
                            int32_t *tokens, int32_t *plen, int32_t *unpacker, int32_t *depth, int32_t *src,
                            uint32_t *mask, hipStream_t stream);
hipError_t launch_tree_mask(const int32_t *unpacker, const int32_t *plen, int B, int W, int L,
                            uint32_t *mask, hipStream_t stream);

// tree attention
struct AttnPlan {
    int nqblk;      // query-row blocks per (request, KV head)
    int nsplit;     // KV-cache splits
    int chunk;      // cache keys per split (multiple of the key tile)
    size_t ws_bytes;
    int qpw;        // 16-row query blocks per wavefront (1 or 2)
    int rows_unit;  // nqblk * rows per workgroup
    int nwave;      // wavefronts per workgroup (4 or 8)
    int ksplit;     // wavefronts sharing one query block's keys of a tile (1 or 2)
};
AttnPlan plan_attention(int dtype, int B, int P_max, int Hq, int Hkv, int D, int S_max);
// paged cache: pools [num_pages, Hkv, page_size, D], block table [B, max_pages]
struct PagedKV {
    const int32_t *block_table;
    int max_pages, page_size;
    int64_t num_pages;
};
// paged != nullptr: k_cache / v_cache are the pools and S_max = max_pages * page_size
hipError_t launch_attention(int dtype, const AttnPlan &plan, const void *q, const void *k_new,
                            const void *v_new, const void *k_cache, const void *v_cache,
                            const int32_t *kv_len, const uint32_t *mask, const int32_t *plen,
                            int B, int P_max, int Hq, int Hkv, int D, int S_max, float scale,
                            void *out, void *ws, hipStream_t stream, const PagedKV *paged = nullptr);

// output projection + argmax
struct LmPlan {
    int rows_pad;   // B * P_max
    int vtile;      // vocabulary columns per workgroup
    int rtile;      // compact rows per workgroup (bf16)
    int variant;    // bf16 tile shape
    int nvt;        // vocabulary tiles
    size_t ws_bytes;
};
LmPlan plan_lm_head(int dtype, int B, int P_max, int K, int V);
hipError_t launch_lm_head(int dtype, const LmPlan &plan, const void *hidden, const int32_t *plen,
                          const void *weight, int B, int P_max, int K, int V, void *logits,
                          int32_t *argmax, void *ws, hipStream_t stream, const int32_t *node_row = nullptr);
// device address of the current device's fixed projection scratch (RD_NOALLOC_SCRATCH_BYTES)
hipError_t noalloc_scratch(void **out);

// unpack gather + accept
hipError_t launch_unpack_accept(const void *packed, void *unpacked, const int32_t *unpacker, int64_t row_bytes,
                                const int32_t *beams, const int32_t *pargmax, int B, int W, int L,
                                int32_t *match_len, int32_t *best_beam, int32_t *accept_len,
                                int32_t *accepted, hipStream_t stream, const int32_t *bwid = nullptr,
                                const int32_t *blen = nullptr);

// unpack folded into the projection: node_row[b*P + p] = output row
// (b*W + w)*L + l of packed row p's first candidate (lowest w), -1 for a row
// no candidate stands for; todo[b*P + j], j < ntodo[b], lists request b's
// other output rows as (row, source row or -1 for zeros), filled afterwards
hipError_t launch_node_rows(const int32_t *unpacker, int B, int W, int L, int32_t *node_row, int2 *todo,
                            int32_t *ntodo, hipStream_t stream);
hipError_t launch_unpack_dups(void *unpacked, const int2 *todo, const int32_t *ntodo, int64_t row_bytes, int B,
                              int W, int L, hipStream_t stream);

// commit of the accepted path (esize = bytes per element)
hipError_t launch_commit(int esize, const int32_t *unpacker, const int32_t *best_beam, const int32_t *accept_len,
                         const void *k_new, const void *v_new, const void *hidden, int B, int W, int L, int Hkv,
                         int D, int K, int S, void *k_cache, void *v_cache, int32_t *kv_len, void *hidden_next,
                         hipStream_t stream, const PagedKV *paged = nullptr);

// stochastic verification (multi-step speculative sampling over the tree)
size_t stochastic_workspace_bytes(int B, int W, int L);
hipError_t launch_stochastic_accept(int dtype, const int32_t *unpacker, const int32_t *plen, const int32_t *ptok,
                                    const void *logits, const float *q, const float *u_accept, const float *u_bonus,
                                    int B, int W, int L, int V, int32_t *best_beam, int32_t *accept_len,
                                    int32_t *accepted, int32_t *path, void *ws, hipStream_t stream);

int device_cu_count();

// tuning knobs (rd_set_knob): 0 = automatic
int knob(int which);
int set_knob(int which, int value);
// debug mode (rd_set_debug / RD_DEBUG): device-side contents are checked before launching
bool debug_checks();
int set_debug(int on);
struct RangeCheck {  // p[0..n) must lie in [lo, hi)
    const int32_t *p;
    int64_t n;
    int lo, hi;
};
struct TableCheck {  // block-table entries of positions below kv_len[b] must lie in [0, num_pages)
    const int32_t *bt, *kv_len;
    int B, max_pages, page_size;
    int64_t num_pages;
};
// runs the checks on `stream` and waits for them: RD_OK, RD_E_CONTENT or RD_E_HIP
int check_contents(hipStream_t stream, const RangeCheck *checks, int n, const TableCheck *table = nullptr);

}  // namespace rd
