// C ABI of librd: argument validation and launch of the step kernels.
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <initializer_list>
#include <mutex>

#include "../../include/rd.h"
#include "rd_internal.h"

namespace rd {

int device_cu_count() {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

}  // namespace rd

namespace {

hipStream_t as_stream(rd_stream_t s) { return static_cast<hipStream_t>(s); }

int hip_status(hipError_t e) { return e == hipSuccess ? RD_OK : RD_E_HIP; }

bool beam_shape_ok(int B, int W, int L) { return B >= 0 && W >= 0 && L >= 0; }
bool beam_shape_supported(int W, int L) { return W <= rd::kMaxBeams && L <= rd::kMaxBeamLen; }

// Debug mode: check the device-side values a call trusts before it launches anything.
int debug_check(rd_stream_t stream, std::initializer_list<rd::RangeCheck> checks,
                const rd::TableCheck *table = nullptr) {
    if (!rd::debug_checks()) return RD_OK;
    return rd::check_contents(as_stream(stream), checks.begin(), static_cast<int>(checks.size()), table);
}

}  // namespace

extern "C" {

const char *rd_status_string(int status) {
    switch (status) {
        case RD_OK: return "RD_OK";
        case RD_E_ARG: return "RD_E_ARG: invalid argument (null pointer, negative or inconsistent size)";
        case RD_E_UNSUPPORTED: return "RD_E_UNSUPPORTED: size or dtype outside the library's limits";
        case RD_E_WORKSPACE: return "RD_E_WORKSPACE: workspace smaller than the size query returned";
        case RD_E_HIP: return "RD_E_HIP: a HIP launch failed";
        case RD_E_CONTENT: return "RD_E_CONTENT: a device-side length, slot or page id is out of range (debug mode)";
        case RD_E_SCRATCH:
            return "RD_E_SCRATCH: the call needs more scratch than the fixed device array holds "
                   "(RD_NOALLOC_SCRATCH_BYTES); use the workspace entry point";
        default: return "unknown rd status";
    }
}

int rd_version(void) { return 100; }

int rd_pack_beams(const int32_t *beams, int B, int W, int L, int32_t *packed_tokens, int32_t *packed_len,
                  int32_t *unpacker, int32_t *packed_depth, int32_t *packed_src, rd_stream_t stream) {
    if (!beam_shape_ok(B, W, L)) return RD_E_ARG;
    if (B == 0 || W == 0 || L == 0) return RD_OK;
    if (!beams || !packed_tokens || !packed_len || !unpacker) return RD_E_ARG;
    if (!beam_shape_supported(W, L)) return RD_E_UNSUPPORTED;
    return hip_status(rd::launch_pack_beams(beams, B, W, L, packed_tokens, packed_len, unpacker, packed_depth,
                                            packed_src, as_stream(stream)));
}

int rd_pack_beams_mask(const int32_t *beams, int B, int W, int L, int32_t *packed_tokens, int32_t *packed_len,
                       int32_t *unpacker, int32_t *packed_depth, int32_t *packed_src, uint32_t *mask,
                       rd_stream_t stream) {
    if (!beam_shape_ok(B, W, L)) return RD_E_ARG;
    if (B == 0 || W == 0 || L == 0) return RD_OK;
    if (!beams || !packed_tokens || !packed_len || !unpacker || !mask) return RD_E_ARG;
    if (!beam_shape_supported(W, L)) return RD_E_UNSUPPORTED;
    return hip_status(rd::launch_pack_mask(beams, nullptr, nullptr, B, W, L, packed_tokens, packed_len, unpacker,
                                           packed_depth, packed_src, mask, as_stream(stream)));
}

int rd_pack_beams_mask_ragged(const int32_t *beams, const int32_t *beam_width, const int32_t *beam_len, int B, int W,
                              int L, int32_t *packed_tokens, int32_t *packed_len, int32_t *unpacker,
                              int32_t *packed_depth, int32_t *packed_src, uint32_t *mask, rd_stream_t stream) {
    if (!beam_shape_ok(B, W, L)) return RD_E_ARG;
    if (B == 0 || W == 0 || L == 0) return RD_OK;
    if (!beams || !beam_width || !beam_len || !packed_tokens || !packed_len || !unpacker || !mask) return RD_E_ARG;
    if (!beam_shape_supported(W, L)) return RD_E_UNSUPPORTED;
    return hip_status(rd::launch_pack_mask(beams, beam_width, beam_len, B, W, L, packed_tokens, packed_len, unpacker,
                                           packed_depth, packed_src, mask, as_stream(stream)));
}

int rd_tree_mask(const int32_t *unpacker, const int32_t *packed_len, int B, int W, int L, uint32_t *mask,
                 rd_stream_t stream) {
    if (!beam_shape_ok(B, W, L)) return RD_E_ARG;
    if (B == 0 || W == 0 || L == 0) return RD_OK;
    if (!unpacker || !packed_len || !mask) return RD_E_ARG;
    if (!beam_shape_supported(W, L)) return RD_E_UNSUPPORTED;
    const int P = W * L;
    const int dbg = debug_check(stream, {{unpacker, static_cast<int64_t>(B) * P, -1, P}, {packed_len, B, 0, P + 1}});
    if (dbg != RD_OK) return dbg;
    return hip_status(rd::launch_tree_mask(unpacker, packed_len, B, W, L, mask, as_stream(stream)));
}

static int attn_check(int dtype, int B, int P_max, int Hq, int Hkv, int D, int S_max) {
    if (B < 0 || P_max < 0 || Hq < 0 || Hkv < 0 || D < 0 || S_max < 0) return RD_E_ARG;
    if (dtype != RD_F32 && dtype != RD_BF16) return RD_E_UNSUPPORTED;
    if (B == 0 || P_max == 0 || Hq == 0) return RD_OK;
    if (Hkv == 0 || Hq % Hkv != 0) return RD_E_ARG;
    if (D != 64 && D != 128) return RD_E_UNSUPPORTED;
    if (P_max > rd::kMaxBeams * rd::kMaxBeamLen) return RD_E_UNSUPPORTED;
    // bf16 kernels address one request's packed rows and one (request, KV
    // head) cache slab through 31-bit buffer offsets
    if (dtype == RD_BF16 && (static_cast<long long>(P_max) * Hkv * D * 2 > 0x7FFFFFFFLL ||
                             static_cast<long long>(S_max) * D * 2 > 0x7FFFFFFFLL))
        return RD_E_UNSUPPORTED;
    return RD_OK;
}

size_t rd_tree_attention_workspace_size(int dtype, int B, int P_max, int Hq, int Hkv, int D, int S_max) {
    if (attn_check(dtype, B, P_max, Hq, Hkv, D, S_max) != RD_OK || B == 0 || P_max == 0 || Hq == 0) return 0;
    return rd::plan_attention(dtype, B, P_max, Hq, Hkv, D, S_max).ws_bytes;
}

int rd_tree_attention(int dtype, const void *q, const void *k_new, const void *v_new, const void *k_cache,
                      const void *v_cache, const int32_t *kv_len, const uint32_t *mask, const int32_t *packed_len,
                      int B, int P_max, int Hq, int Hkv, int D, int S_max, float scale, void *out, void *ws,
                      size_t ws_bytes, rd_stream_t stream) {
    const int chk = attn_check(dtype, B, P_max, Hq, Hkv, D, S_max);
    if (chk != RD_OK) return chk;
    if (B == 0 || P_max == 0 || Hq == 0) return RD_OK;
    if (!q || !k_new || !v_new || !kv_len || !mask || !packed_len || !out) return RD_E_ARG;
    if (S_max > 0 && (!k_cache || !v_cache)) return RD_E_ARG;
    if (!(scale >= 0.f) || !(scale <= 3.4e38f)) return RD_E_ARG;  // finite, non-negative (rejects NaN)
    const rd::AttnPlan plan = rd::plan_attention(dtype, B, P_max, Hq, Hkv, D, S_max);
    if (ws_bytes < plan.ws_bytes || (plan.ws_bytes > 0 && !ws)) return RD_E_WORKSPACE;
    const int dbg = debug_check(stream, {{kv_len, B, 0, S_max + 1}, {packed_len, B, 0, P_max + 1}});
    if (dbg != RD_OK) return dbg;
    return hip_status(rd::launch_attention(dtype, plan, q, k_new, v_new, k_cache, v_cache, kv_len, mask, packed_len,
                                           B, P_max, Hq, Hkv, D, S_max, scale, out, ws, as_stream(stream)));
}

int rd_tree_attention_paged(int dtype, const void *q, const void *k_new, const void *v_new, const void *k_pages,
                            const void *v_pages, int64_t num_pages, int page_size, const int32_t *block_table,
                            int max_pages, const int32_t *kv_len, const uint32_t *mask, const int32_t *packed_len,
                            int B, int P_max, int Hq, int Hkv, int D, float scale, void *out, void *ws,
                            size_t ws_bytes, rd_stream_t stream) {
    if (num_pages < 0 || page_size < 1 || max_pages < 0) return RD_E_ARG;
    const long long S = static_cast<long long>(max_pages) * page_size;
    if (S > 0x7FFFFFFFLL) return RD_E_UNSUPPORTED;
    const int chk = attn_check(dtype, B, P_max, Hq, Hkv, D, static_cast<int>(S));
    if (chk != RD_OK) return chk;
    if (B == 0 || P_max == 0 || Hq == 0) return RD_OK;
    if (!q || !k_new || !v_new || !kv_len || !mask || !packed_len || !out) return RD_E_ARG;
    if (S > 0 && (!k_pages || !v_pages || !block_table || num_pages < 1)) return RD_E_ARG;
    if (dtype == RD_BF16 && page_size % 64 != 0) return RD_E_UNSUPPORTED;  // a key tile must not cross a page
    if (!(scale >= 0.f) || !(scale <= 3.4e38f)) return RD_E_ARG;
    const rd::AttnPlan plan = rd::plan_attention(dtype, B, P_max, Hq, Hkv, D, static_cast<int>(S));
    if (ws_bytes < plan.ws_bytes || (plan.ws_bytes > 0 && !ws)) return RD_E_WORKSPACE;
    const rd::PagedKV pk{block_table, max_pages, page_size, num_pages > 0 ? num_pages : 1};
    const rd::TableCheck tc{block_table, kv_len, B, max_pages, page_size, num_pages};
    const int dbg = debug_check(stream, {{kv_len, B, 0, static_cast<int>(S) + 1}, {packed_len, B, 0, P_max + 1}},
                                S > 0 ? &tc : nullptr);
    if (dbg != RD_OK) return dbg;
    return hip_status(rd::launch_attention(dtype, plan, q, k_new, v_new, k_pages, v_pages, kv_len, mask, packed_len,
                                           B, P_max, Hq, Hkv, D, static_cast<int>(S), scale, out, ws,
                                           as_stream(stream), &pk));
}

static int lm_check(int dtype, int B, int P_max, int K, int V) {
    if (B < 0 || P_max < 0 || K < 0 || V < 0) return RD_E_ARG;
    if (dtype != RD_F32 && dtype != RD_BF16) return RD_E_UNSUPPORTED;
    if (B == 0 || P_max == 0) return RD_OK;
    if (K == 0 || V == 0) return RD_E_ARG;
    if (dtype == RD_BF16 && K % 8 != 0) return RD_E_UNSUPPORTED;
    if (static_cast<long long>(B) * P_max > (1LL << 30)) return RD_E_UNSUPPORTED;
    // bf16 kernels address the hidden rows and each wavefront's weight rows
    // through 31-bit buffer offsets
    if (dtype == RD_BF16 && static_cast<long long>(B) * P_max * K * 2 > 0x7FFFFFFFLL) return RD_E_UNSUPPORTED;
    return RD_OK;
}

size_t rd_lm_head_workspace_size(int dtype, int B, int P_max, int K, int V) {
    if (lm_check(dtype, B, P_max, K, V) != RD_OK || B == 0 || P_max == 0) return 0;
    return rd::plan_lm_head(dtype, B, P_max, K, V).ws_bytes;
}

int rd_lm_head_argmax(int dtype, const void *hidden, const int32_t *packed_len, const void *weight, int B,
                      int P_max, int K, int V, void *logits, int32_t *argmax, void *ws, size_t ws_bytes,
                      rd_stream_t stream) {
    const int chk = lm_check(dtype, B, P_max, K, V);
    if (chk != RD_OK) return chk;
    if (B == 0 || P_max == 0) return RD_OK;
    if (!hidden || !weight || !argmax) return RD_E_ARG;
    const rd::LmPlan plan = rd::plan_lm_head(dtype, B, P_max, K, V);
    if (ws_bytes < plan.ws_bytes || !ws) return RD_E_WORKSPACE;
    const int dbg = debug_check(stream, {{packed_len, packed_len ? B : 0, 0, P_max + 1}});
    if (dbg != RD_OK) return dbg;
    return hip_status(rd::launch_lm_head(dtype, plan, hidden, packed_len, weight, B, P_max, K, V, logits, argmax,
                                         ws, as_stream(stream)));
}

// the unpacked projection's workspace: the projection's, then per packed row its
// output row, per candidate one entry of the fill list, per request the list length
static size_t ws_round(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
static size_t unpack_ws_bytes(const rd::LmPlan &plan, int B, int W, int L) {
    const size_t n = static_cast<size_t>(B) * W * L;
    return plan.ws_bytes + ws_round(n * sizeof(int32_t)) + ws_round(n * sizeof(int2)) + ws_round(B * sizeof(int32_t));
}

static int lm_unpack_check(int dtype, int B, int W, int L, int K, int V) {
    if (!beam_shape_ok(B, W, L)) return RD_E_ARG;
    if (B == 0 || W == 0 || L == 0) return RD_OK;
    if (!beam_shape_supported(W, L)) return RD_E_UNSUPPORTED;
    return lm_check(dtype, B, W * L, K, V);
}

size_t rd_lm_head_argmax_unpack_workspace_size(int dtype, int B, int W, int L, int K, int V) {
    if (lm_unpack_check(dtype, B, W, L, K, V) != RD_OK || B == 0 || W == 0 || L == 0) return 0;
    return unpack_ws_bytes(rd::plan_lm_head(dtype, B, W * L, K, V), B, W, L);
}

int rd_lm_head_argmax_unpack(int dtype, const void *hidden, const int32_t *packed_len, const void *weight,
                             const int32_t *unpacker, int B, int W, int L, int K, int V, void *unpacked,
                             int32_t *argmax, void *ws, size_t ws_bytes, rd_stream_t stream) {
    const int chk = lm_unpack_check(dtype, B, W, L, K, V);
    if (chk != RD_OK) return chk;
    if (B == 0 || W == 0 || L == 0) return RD_OK;
    if (!hidden || !weight || !unpacker || !unpacked || !argmax) return RD_E_ARG;
    const int P = W * L;
    const rd::LmPlan plan = rd::plan_lm_head(dtype, B, P, K, V);
    if (!ws || ws_bytes < unpack_ws_bytes(plan, B, W, L)) return RD_E_WORKSPACE;
    const int dbg = debug_check(stream, {{packed_len, packed_len ? B : 0, 0, P + 1},
                                         {unpacker, B * P, -1, P}});
    if (dbg != RD_OK) return dbg;
    const size_t n = static_cast<size_t>(B) * P;
    char *w = static_cast<char *>(ws) + plan.ws_bytes;
    int32_t *node_row = reinterpret_cast<int32_t *>(w);
    int2 *todo = reinterpret_cast<int2 *>(w + ws_round(n * sizeof(int32_t)));
    int32_t *ntodo = reinterpret_cast<int32_t *>(w + ws_round(n * sizeof(int32_t)) + ws_round(n * sizeof(int2)));
    const hipStream_t s = as_stream(stream);
    hipError_t err = rd::launch_node_rows(unpacker, B, W, L, node_row, todo, ntodo, s);
    if (err == hipSuccess)
        err = rd::launch_lm_head(dtype, plan, hidden, packed_len, weight, B, P, K, V, unpacked, argmax, ws, s,
                                 node_row);
    if (err == hipSuccess)
        err = rd::launch_unpack_dups(unpacked, todo, ntodo, static_cast<int64_t>(V) * (dtype == RD_BF16 ? 2 : 4), B,
                                     W, L, s);
    return hip_status(err);
}

int rd_lm_head_argmax_noalloc(int dtype, const void *hidden, const int32_t *packed_len, const void *weight, int B,
                              int P_max, int K, int V, void *logits, int32_t *argmax, rd_stream_t stream) {
    const int chk = lm_check(dtype, B, P_max, K, V);
    if (chk != RD_OK) return chk;
    if (B == 0 || P_max == 0) return RD_OK;
    if (!hidden || !weight || !argmax) return RD_E_ARG;
    const rd::LmPlan plan = rd::plan_lm_head(dtype, B, P_max, K, V);
    if (plan.ws_bytes > RD_NOALLOC_SCRATCH_BYTES) return RD_E_SCRATCH;
    void *ws = nullptr;
    if (rd::noalloc_scratch(&ws) != hipSuccess) return RD_E_HIP;
    const int dbg = debug_check(stream, {{packed_len, packed_len ? B : 0, 0, P_max + 1}});
    if (dbg != RD_OK) return dbg;
    return hip_status(rd::launch_lm_head(dtype, plan, hidden, packed_len, weight, B, P_max, K, V, logits, argmax,
                                         ws, as_stream(stream)));
}

}  // extern "C"

namespace {

int unpack_accept(const int32_t *beams, const int32_t *bwid, const int32_t *blen, const int32_t *unpacker,
                  const int32_t *packed_argmax, const void *packed, void *unpacked, int dtype, int64_t row_len, int B,
                  int W, int L, int32_t *match_len, int32_t *best_beam, int32_t *accept_len,
                  int32_t *accepted_tokens, rd_stream_t stream) {
    if (!beam_shape_ok(B, W, L) || row_len < 0) return RD_E_ARG;
    if (B == 0 || W == 0 || L == 0) return RD_OK;
    if (!beams || !unpacker || !packed_argmax || !match_len || !best_beam || !accept_len || !accepted_tokens)
        return RD_E_ARG;
    if (!beam_shape_supported(W, L)) return RD_E_UNSUPPORTED;
    if (dtype != RD_F32 && dtype != RD_BF16) return RD_E_UNSUPPORTED;
    hipStream_t s = as_stream(stream);
    int64_t row_bytes = 0;
    if (packed && unpacked && row_len > 0) {
        row_bytes = row_len * (dtype == RD_F32 ? 4 : 2);
        const int64_t rows = static_cast<int64_t>(B) * W * L;
        const int64_t chunks = (row_bytes + 1023) / 1024;  // upper bound on blocks per row
        if (rows * chunks * 256 >= (1LL << 32)) return RD_E_UNSUPPORTED;
    }
    const int dbg = debug_check(stream, {{unpacker, static_cast<int64_t>(B) * W * L, -1, W * L}});
    if (dbg != RD_OK) return dbg;
    return hip_status(rd::launch_unpack_accept(row_bytes ? packed : nullptr, row_bytes ? unpacked : nullptr, unpacker,
                                               row_bytes, beams, packed_argmax, B, W, L, match_len, best_beam,
                                               accept_len, accepted_tokens, s, bwid, blen));
}

}  // namespace

extern "C" {

int rd_unpack_accept(const int32_t *beams, const int32_t *unpacker, const int32_t *packed_argmax, const void *packed,
                     void *unpacked, int dtype, int64_t row_len, int B, int W, int L, int32_t *match_len,
                     int32_t *best_beam, int32_t *accept_len, int32_t *accepted_tokens, rd_stream_t stream) {
    return unpack_accept(beams, nullptr, nullptr, unpacker, packed_argmax, packed, unpacked, dtype, row_len, B, W, L,
                         match_len, best_beam, accept_len, accepted_tokens, stream);
}

int rd_unpack_accept_ragged(const int32_t *beams, const int32_t *beam_width, const int32_t *beam_len,
                            const int32_t *unpacker, const int32_t *packed_argmax, const void *packed, void *unpacked,
                            int dtype, int64_t row_len, int B, int W, int L, int32_t *match_len, int32_t *best_beam,
                            int32_t *accept_len, int32_t *accepted_tokens, rd_stream_t stream) {
    if (B > 0 && W > 0 && L > 0 && (!beam_width || !beam_len)) return RD_E_ARG;
    return unpack_accept(beams, beam_width, beam_len, unpacker, packed_argmax, packed, unpacked, dtype, row_len, B, W,
                         L, match_len, best_beam, accept_len, accepted_tokens, stream);
}

size_t rd_stochastic_accept_workspace_size(int B, int W, int L) {
    if (!beam_shape_ok(B, W, L) || !beam_shape_supported(W, L)) return 0;
    return rd::stochastic_workspace_bytes(B, W, L);
}

int rd_stochastic_accept(int dtype, const int32_t *unpacker, const int32_t *packed_len, const int32_t *packed_tokens,
                         const void *logits, const float *q, const float *u_accept, const float *u_bonus, int B,
                         int W, int L, int V, int32_t *best_beam, int32_t *accept_len, int32_t *accepted_tokens,
                         int32_t *path, void *ws, size_t ws_bytes, rd_stream_t stream) {
    if (!beam_shape_ok(B, W, L) || V < 0) return RD_E_ARG;
    if (B == 0 || W == 0 || L == 0) return RD_OK;
    if (V == 0 || !unpacker || !packed_len || !packed_tokens || !logits || !q || !u_accept || !u_bonus ||
        !best_beam || !accept_len || !accepted_tokens)
        return RD_E_ARG;
    if (!beam_shape_supported(W, L)) return RD_E_UNSUPPORTED;
    if (dtype != RD_F32 && dtype != RD_BF16) return RD_E_UNSUPPORTED;
    if (ws_bytes < rd::stochastic_workspace_bytes(B, W, L) || !ws) return RD_E_WORKSPACE;
    const int dbg = debug_check(stream, {{unpacker, static_cast<int64_t>(B) * W * L, -1, W * L},
                                         {packed_len, B, 0, W * L + 1}});
    if (dbg != RD_OK) return dbg;
    return hip_status(rd::launch_stochastic_accept(dtype, unpacker, packed_len, packed_tokens, logits, q, u_accept,
                                                   u_bonus, B, W, L, V, best_beam, accept_len, accepted_tokens, path,
                                                   ws, as_stream(stream)));
}

int rd_commit_accepted(int dtype, const int32_t *unpacker, const int32_t *best_beam, const int32_t *accept_len,
                       const void *k_new, const void *v_new, const void *hidden, int B, int W, int L, int Hkv,
                       int D, int K, int S_max, void *k_cache, void *v_cache, int32_t *kv_len, void *hidden_next,
                       rd_stream_t stream) {
    if (!beam_shape_ok(B, W, L) || Hkv < 1 || D < 1 || K < 0 || S_max < 0) return RD_E_ARG;
    if (B == 0 || W == 0 || L == 0) return RD_OK;
    if (!unpacker || !best_beam || !accept_len || !k_new || !v_new || !k_cache || !v_cache || !kv_len)
        return RD_E_ARG;
    if ((hidden != nullptr) != (hidden_next != nullptr) || (hidden && K < 1)) return RD_E_ARG;
    if (!beam_shape_supported(W, L)) return RD_E_UNSUPPORTED;
    if (dtype != RD_F32 && dtype != RD_BF16) return RD_E_UNSUPPORTED;
    const int64_t esize = dtype == RD_F32 ? 4 : 2;
    // copy units (2 bytes at the narrowest) of one request must index in 32 bits
    const int64_t units = (2 * static_cast<int64_t>(Hkv) * L * D + (hidden ? K : 0)) * esize / 2;
    if (units >= (1LL << 30)) return RD_E_UNSUPPORTED;
    const int dbg = debug_check(stream, {{unpacker, static_cast<int64_t>(B) * W * L, -1, W * L},
                                         {kv_len, B, 0, S_max + 1}});
    if (dbg != RD_OK) return dbg;
    return hip_status(rd::launch_commit(static_cast<int>(esize), unpacker, best_beam, accept_len, k_new, v_new,
                                        hidden, B, W, L, Hkv, D, K, S_max, k_cache, v_cache, kv_len, hidden_next,
                                        as_stream(stream)));
}

int rd_commit_accepted_paged(int dtype, const int32_t *unpacker, const int32_t *best_beam, const int32_t *accept_len,
                             const void *k_new, const void *v_new, const void *hidden, int B, int W, int L, int Hkv,
                             int D, int K, void *k_pages, void *v_pages, int64_t num_pages, int page_size,
                             const int32_t *block_table, int max_pages, int32_t *kv_len, void *hidden_next,
                             rd_stream_t stream) {
    if (!beam_shape_ok(B, W, L) || Hkv < 1 || D < 1 || K < 0 || num_pages < 0 || page_size < 1 || max_pages < 0)
        return RD_E_ARG;
    if (B == 0 || W == 0 || L == 0) return RD_OK;
    if (!unpacker || !best_beam || !accept_len || !k_new || !v_new || !k_pages || !v_pages || !block_table ||
        !kv_len || num_pages < 1)
        return RD_E_ARG;
    if ((hidden != nullptr) != (hidden_next != nullptr) || (hidden && K < 1)) return RD_E_ARG;
    if (!beam_shape_supported(W, L)) return RD_E_UNSUPPORTED;
    if (dtype != RD_F32 && dtype != RD_BF16) return RD_E_UNSUPPORTED;
    const long long S = static_cast<long long>(max_pages) * page_size;
    if (S > 0x7FFFFFFFLL) return RD_E_UNSUPPORTED;
    const int64_t esize = dtype == RD_F32 ? 4 : 2;
    const int64_t units = (2 * static_cast<int64_t>(Hkv) * L * D + (hidden ? K : 0)) * esize / 2;
    if (units >= (1LL << 30)) return RD_E_UNSUPPORTED;
    const rd::PagedKV pk{block_table, max_pages, page_size, num_pages};
    const int dbg = debug_check(stream, {{unpacker, static_cast<int64_t>(B) * W * L, -1, W * L},
                                         {kv_len, B, 0, static_cast<int>(S) + 1}});
    if (dbg != RD_OK) return dbg;
    return hip_status(rd::launch_commit(static_cast<int>(esize), unpacker, best_beam, accept_len, k_new, v_new,
                                        hidden, B, W, L, Hkv, D, K, static_cast<int>(S), k_pages, v_pages, kv_len,
                                        hidden_next, as_stream(stream), &pk));
}

}  // extern "C"
