/*
 * rd.h -- C ABI of the ReDrafter verification-step library (librd.so, gfx950).
 *
 * One verification step of Recurrent Drafting checks the W beam-search
 * candidates of length L of each of B requests against the target model in a
 * single pass: (1) shared prefixes are removed into a packed token tree with
 * an unpacker index and a tree-causal mask, (2) the packed tokens attend to
 * the request's KV cache and their tree ancestors, (3) the outputs are
 * projected to logits, reduced to the target's greedy choice and unpacked to
 * [B,W,L,V], (4) the beam with the longest prefix that agrees with the target
 * is accepted together with one bonus token.
 *
 * Sources, cited by page title and section:
 *   [TRT]   "ReDrafter in NVIDIA TensorRT-LLM" blog: intro; "Inflight-batching
 *           Compatible Engine"; "Implementing in-Engine Validation and
 *           Drafting" (the PyTorch `unpack` and TensorRT-LLM `_unpack_beams`
 *           listings).
 *   [NEWS]  Apple/NVIDIA ReDrafter news article: "RNN draft model", "Dynamic
 *           tree attention", greedy-decoding benchmark paragraph.
 *   [PAPER] "Recurrent Drafter for Fast Speculative Decoding in Large Language
 *           Models", abstract point (2).
 *   [SURV]  "Accelerating LLM inference with speculative decoding" survey,
 *           SpecInfer "Token Tree Verifier".
 *
 * Conventions shared by every entry point
 *   - Pointers marked (dev) are device memory owned by the caller; the
 *     library never allocates, frees or retains them past the call.  Arrays
 *     are dense and row-major in the shapes given; int32 unless stated.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *     null stream) and returns without synchronising the host.  Results are
 *     valid once the stream reaches that point.
 *   - P_max == W*L is the static packed width: no call reads packed lengths
 *     back to the host.
 *   - Status: RD_OK, or a negative code from host-side validation made
 *     before anything is launched (RD_E_ARG: null required pointer, negative
 *     size, inconsistent shape; RD_E_UNSUPPORTED: size or dtype outside the
 *     limits below; RD_E_WORKSPACE: workspace smaller than its query), or
 *     RD_E_HIP when a launch fails.
 *   - Empty inputs (any of B, W, L == 0) return RD_OK with nothing launched:
 *     [TRT] "Inflight-batching Compatible Engine" requires every operator on
 *     the generation path to accept empty tensors.
 *   - Device-side contents (kv_len <= S_max, unpacker values in [0,P_max))
 *     are trusted as produced by rd_pack_beams; kernels clamp every index
 *     they derive from them so a bad value cannot address outside the
 *     arrays, but the results are then unspecified.  Debug mode
 *     (rd_set_debug) checks them first and returns RD_E_CONTENT instead.
 *   - Results are deterministic: identical inputs give bit-identical outputs
 *     (no floating-point atomics, fixed reduction orders).
 *   - The library keeps no state between calls and is safe to call from
 *     several host threads on different streams.
 */
#ifndef RD_H
#define RD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *rd_stream_t; /* hipStream_t */

enum rd_status_code {
    RD_OK = 0,
    RD_E_ARG = -1,
    RD_E_UNSUPPORTED = -2,
    RD_E_WORKSPACE = -3,
    RD_E_HIP = -4,
    RD_E_CONTENT = -5, /* debug mode only: a device-side value is out of range */
    RD_E_SCRATCH = -6  /* rd_lm_head_argmax_noalloc: sizes need more than its fixed scratch */
};

enum rd_dtype {
    RD_F32 = 0,  /* IEEE binary32 */
    RD_BF16 = 1  /* bfloat16; computed with fp32 accumulation */
};

#define RD_MAX_BEAMS 64      /* W limit: one wavefront lane per beam */
#define RD_MAX_BEAM_LEN 16   /* L limit */

/* Human-readable name of a status code (static storage). */
const char *rd_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int rd_version(void);

/*
 * Tuning knobs (for tests and measurements; not needed in production).
 * Each forces a choice the library otherwise makes itself; 0 restores the
 * automatic choice.  Knobs are process-wide, read by every later call
 * (workspace-size queries included: query after setting), and not
 * synchronised with calls already running on other host threads.
 *   RD_KNOB_ATTN_SPLITS  n >= 1: split each (request, KV head)'s cache
 *                        into n parts (clamped to the key tiles), merged
 *                        by log-sum-exp; bf16 attention only.
 *   RD_KNOB_ATTN_FEWROW  1: lane-interleaved eight-wavefront shape for at
 *                        most 64 rows per (request, KV head); 2: the
 *                        four-wavefront shape.  bf16 attention only.
 *   RD_KNOB_LM_SHAPE     1: the few-row projection tile shape; 2: the
 *                        many-row shape.  bf16 projection only.
 * Returns the previous value, or RD_E_ARG for an unknown knob or a
 * negative value.
 */
enum rd_knob {
    RD_KNOB_ATTN_SPLITS = 1,
    RD_KNOB_ATTN_FEWROW = 2,
    RD_KNOB_LM_SHAPE = 3,
    RD_KNOB_COUNT = 4
};
int rd_set_knob(int knob, int value);

/*
 * Debug mode (also switched on by RD_DEBUG=1 in the environment when the
 * library is first used).  Every entry point then checks, before launching
 * its kernels, the device-side values it otherwise trusts: kv_len in
 * [0, S_max], packed_len in [0, P_max], unpacker slots in [-1, P_max), and
 * the block-table entries of every cached position in [0, num_pages).  The
 * checks run on `stream`, the host waits for them, and a bad value makes
 * the call return RD_E_CONTENT with nothing else launched.  Debug mode
 * therefore synchronises the host on every call.  Returns the previous
 * setting (0 or 1).
 */
int rd_set_debug(int on);

/*
 * Step 1 -- pack: remove shared prefixes across each request's beams.
 * [NEWS] "Dynamic tree attention", [PAPER] abstract (2): beams share
 * prefixes; each distinct prefix beams[b,w,0..l] is verified once.
 * [TRT] PyTorch `unpack`: unpacker[b,w,l] indexes dimension 1 of the packed
 * tensor.  Packed slots are numbered in the order a beam-major scan first
 * meets each prefix, so a parent precedes its children.
 *
 *   beams         (dev) [B,W,L]  token ids (any int32 values)
 *   packed_tokens (dev) [B,P_max] token of each slot, -1 past packed_len
 *   packed_len    (dev) [B]      number of distinct prefixes of request b
 *   unpacker      (dev) [B,W,L]  slot of candidate (w,l), in [0,packed_len)
 *   packed_depth  (dev) [B,P_max] depth l of each slot, -1 padding; may be NULL
 *   packed_src    (dev) [B,P_max] w*L+l of each slot's first occurrence, -1
 *                                 padding; may be NULL
 * Limits: W <= RD_MAX_BEAMS, L <= RD_MAX_BEAM_LEN.
 */
int rd_pack_beams(const int32_t *beams, int B, int W, int L,
                  int32_t *packed_tokens, int32_t *packed_len, int32_t *unpacker,
                  int32_t *packed_depth, int32_t *packed_src, rd_stream_t stream);

/*
 * Step 1b -- tree-causal mask.  [SURV] SpecInfer "Token Tree Verifier": one
 * topology-aware causal mask lets every path of the tree be evaluated in one
 * kernel.  Bit q of row p is set iff slot q is slot p or one of its
 * ancestors; rows and columns at or past packed_len are zero.
 *
 *   unpacker, packed_len (dev) as produced by rd_pack_beams
 *   mask (dev) uint32 [B,P_max,ceil(P_max/32)]: bit (q%32) of word q/32.
 */
int rd_tree_mask(const int32_t *unpacker, const int32_t *packed_len, int B, int W, int L,
                 uint32_t *mask, rd_stream_t stream);

/*
 * Steps 1 and 1b in one launch: exactly rd_pack_beams followed by
 * rd_tree_mask on its outputs (same arguments, same results), for callers
 * that want both; the mask is built from the unpacker while it is still in
 * on-chip memory.
 */
int rd_pack_beams_mask(const int32_t *beams, int B, int W, int L,
                       int32_t *packed_tokens, int32_t *packed_len, int32_t *unpacker,
                       int32_t *packed_depth, int32_t *packed_src, uint32_t *mask,
                       rd_stream_t stream);

/*
 * Steps 1 + 1b for a ragged batch.  [TRT] "Inflight-batching Compatible
 * Engine": the requests of one batch differ in shape.  Request b has
 * beam_width[b] <= W beams of beam_len[b] <= L tokens (dev int32 [B] each,
 * clamped to [0,W] / [0,L]) in the top-left corner of its [W,L] slab of
 * beams; the rest is padding.  Padding candidates open no slot and get
 * unpacker -1; everything else is exactly rd_pack_beams_mask on the request's
 * [beam_width[b], beam_len[b]] sub-array, with packed_src still w*L+l in the
 * padded slab.  A request with no beam or no position has packed_len 0.
 */
int rd_pack_beams_mask_ragged(const int32_t *beams, const int32_t *beam_width,
                              const int32_t *beam_len, int B, int W, int L,
                              int32_t *packed_tokens, int32_t *packed_len, int32_t *unpacker,
                              int32_t *packed_depth, int32_t *packed_src, uint32_t *mask,
                              rd_stream_t stream);

/* Bytes of device workspace rd_tree_attention needs for these sizes (may be 0). */
size_t rd_tree_attention_workspace_size(int dtype, int B, int P_max, int Hq, int Hkv, int D,
                                        int S_max);

/*
 * Step 2 -- tree attention.  [TRT] intro and FAQ: the target verifies draft
 * tokens from several paths at once with tree-style attention; [NEWS]
 * "Dynamic tree attention": deduplication only removes repeated work, so
 * packed slot p = unpacker[b,w,l] must yield the output of causal
 * attention over beam w alone.  For packed query p < packed_len[b] and
 * head h, with KV head g = h / (Hq/Hkv): keys are k_cache[b,g,0:kv_len[b]]
 * (all visible) followed by k_new[b,q,g] for every slot q whose bit is set
 * in mask row p; softmax(q.k * scale) weights the matching values.
 *
 *   dtype        RD_BF16 (fp32 softmax and accumulation, bf16 output) or RD_F32
 *   q       (dev) [B,P_max,Hq,D]   packed queries (already position-encoded)
 *   k_new, v_new (dev) [B,P_max,Hkv,D] packed keys/values
 *   k_cache, v_cache (dev) [B,Hkv,S_max,D]
 *   kv_len  (dev) [B]  cached tokens of request b, 0 <= kv_len[b] <= S_max
 *   mask, packed_len (dev) from rd_tree_mask / rd_pack_beams
 *   scale   softmax scale, finite and >= 0; 0 selects 1/sqrt(D)
 *   out     (dev) [B,P_max,Hq,D]  rows at or past packed_len are written as 0
 *   ws      (dev) workspace of ws_bytes >= rd_tree_attention_workspace_size()
 * Limits: D in {64,128}, Hq % Hkv == 0, P_max <= RD_MAX_BEAMS*RD_MAX_BEAM_LEN.
 */
int rd_tree_attention(int dtype, const void *q, const void *k_new, const void *v_new,
                      const void *k_cache, const void *v_cache, const int32_t *kv_len,
                      const uint32_t *mask, const int32_t *packed_len,
                      int B, int P_max, int Hq, int Hkv, int D, int S_max, float scale,
                      void *out, void *ws, size_t ws_bytes, rd_stream_t stream);

/*
 * Step 2 over a paged KV cache.  [TRT] intro: the engine keeps its KV cache
 * in pages (paged KV caching).  Identical to rd_tree_attention except where
 * cached keys come from: key t (< kv_len[b]) of request b is row
 * t % page_size of page block_table[b, t / page_size] in the pools
 *   k_pages, v_pages (dev) [num_pages, Hkv, page_size, D] in dtype.
 *   block_table (dev) int32 [B, max_pages]; entries past a request's
 *           kv_len are not read; page ids are clamped to [0, num_pages).
 *   kv_len  (dev) [B], clamped to max_pages * page_size.
 * Pages may be shared between requests (a common prefix).  Workspace:
 * rd_tree_attention_workspace_size(dtype, B, P_max, Hq, Hkv, D,
 * max_pages * page_size).  With the same keys and values the results equal
 * rd_tree_attention's.
 * Limits: as rd_tree_attention; for RD_BF16 page_size must be a multiple of
 * 64 (RD_E_UNSUPPORTED otherwise); RD_E_ARG for page_size < 1, negative
 * num_pages or max_pages, or null pools/table when max_pages > 0.
 */
int rd_tree_attention_paged(int dtype, const void *q, const void *k_new, const void *v_new,
                            const void *k_pages, const void *v_pages, int64_t num_pages,
                            int page_size, const int32_t *block_table, int max_pages,
                            const int32_t *kv_len, const uint32_t *mask, const int32_t *packed_len,
                            int B, int P_max, int Hq, int Hkv, int D, float scale,
                            void *out, void *ws, size_t ws_bytes, rd_stream_t stream);

/* Bytes of device workspace rd_lm_head_argmax needs for these sizes. */
size_t rd_lm_head_workspace_size(int dtype, int B, int P_max, int K, int V);

/*
 * Step 3 -- output projection and greedy target token.  [NEWS] greedy
 * decoding: the target's choice at every packed position is the argmax of
 * hidden . weight^T, taken on the fp32 accumulators (never on rounded
 * logits), lowest vocabulary id on ties.  Only rows p < packed_len[b] are
 * computed.
 *
 *   hidden  (dev) [B,P_max,K]  (dtype)
 *   packed_len (dev) [B], or NULL meaning every row is valid
 *   weight  (dev) [V,K]  (nn.Linear layout, dtype)
 *   logits  (dev) [B,P_max,V] in dtype, or NULL to skip writing them; rows
 *           past packed_len are left untouched
 *   argmax  (dev) [B,P_max]  -1 past packed_len
 *   ws      (dev) workspace of ws_bytes >= rd_lm_head_workspace_size()
 * Limits: K % 8 == 0 for RD_BF16.
 */
int rd_lm_head_argmax(int dtype, const void *hidden, const int32_t *packed_len,
                      const void *weight, int B, int P_max, int K, int V,
                      void *logits, int32_t *argmax, void *ws, size_t ws_bytes,
                      rd_stream_t stream);

/*
 * rd_lm_head_argmax for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and limits as rd_lm_head_argmax, but
 * no workspace: the argmax partials go to a fixed array of
 * RD_NOALLOC_SCRATCH_BYTES that the library holds in device memory on every
 * device it runs on, for the life of the process.  The call allocates
 * nothing and frees nothing.
 *   - RD_E_SCRATCH when rd_lm_head_workspace_size(dtype, B, P_max, K, V)
 *     exceeds RD_NOALLOC_SCRATCH_BYTES (nothing is launched).  32 MiB holds
 *     e.g. B*P_max = 32768 rows at V = 32000, or 4096 rows at V = 128256.
 *   - Every call on one device shares that device's array and leaves its
 *     contents behind; the kernels overwrite every partial they read, so
 *     nothing needs clearing.  Calls that overlap on one device (two
 *     streams, or two host threads) race on the array: serialise them.
 *   - The first call on a device looks up the array's device address
 *     (hipGetSymbolAddress) with that device current.
 */
#define RD_NOALLOC_SCRATCH_BYTES (32u << 20)
int rd_lm_head_argmax_noalloc(int dtype, const void *hidden, const int32_t *packed_len,
                              const void *weight, int B, int P_max, int K, int V,
                              void *logits, int32_t *argmax, rd_stream_t stream);

/*
 * Steps 3 and 3b together: rd_lm_head_argmax with the unpack gather of the
 * logits ([TRT] PyTorch `unpack`: unpacked[b,w,l,:] = logits[b,
 * unpacker[b,w,l], :]) folded into it.  Each computed logits row is stored
 * once, straight into the output row of the first candidate it stands for
 * (lowest beam w); the node's other candidates are copied from that row
 * afterwards, and padding candidates (unpacker -1) get zeros.  The packed
 * [B,W*L,V] logits are never written and read back, so with little prefix
 * sharing the gather costs almost nothing.  unpacked and argmax equal, bit
 * for bit, rd_lm_head_argmax (P_max = W*L) followed by rd_unpack_accept's
 * gather; the accept then runs as rd_unpack_accept with packed = NULL.
 *
 *   hidden, packed_len, weight, argmax: as rd_lm_head_argmax, P_max = W*L
 *   unpacker (dev) [B,W,L]: from rd_pack_beams* (values in [-1, W*L))
 *   unpacked (dev) [B,W,L,V] in dtype, written in full
 *   ws      (dev) workspace of ws_bytes >= rd_lm_head_argmax_unpack_workspace_size()
 * Launches: the first-candidate table (one workgroup per request), the
 * projection, the argmax reduction and the duplicate-row copy, in order on
 * stream.  Limits: those of rd_lm_head_argmax, W <= RD_MAX_BEAMS,
 * L <= RD_MAX_BEAM_LEN.  B, W or L = 0 is a no-op.
 */
size_t rd_lm_head_argmax_unpack_workspace_size(int dtype, int B, int W, int L, int K, int V);
int rd_lm_head_argmax_unpack(int dtype, const void *hidden, const int32_t *packed_len,
                             const void *weight, const int32_t *unpacker, int B, int W, int L,
                             int K, int V, void *unpacked, int32_t *argmax, void *ws,
                             size_t ws_bytes, rd_stream_t stream);

/*
 * Steps 3b and 4 -- unpack and greedy accept.
 * Unpack ([TRT] PyTorch `unpack` / TensorRT-LLM `_unpack_beams`):
 *   unpacked[b,w,l,:] = packed[b, unpacker[b,w,l], :] with rows of row_len
 *   elements of dtype; skipped when packed or unpacked is NULL.
 * Accept ([TRT] intro: verify, then accept the best path before the next
 * drafting round; [NEWS] greedy decoding; [NEWS] "RNN draft model": beam
 * position 0 is the target's own initial token):
 *   a[w,l] = packed_argmax[b, unpacker[b,w,l]];
 *   match_len[b,w] = largest n <= L-1 with beams[b,w,j+1] == a[w,j], j < n;
 *   best_beam[b]   = lowest w with the largest match_len;
 *   accept_len[b]  = n = match_len[b,best];
 *   accepted_tokens[b,:] = beams[b,best,1..n], then a[best,n], then -1.
 *
 *   beams, unpacker (dev) [B,W,L]; packed_argmax (dev) [B,P_max]
 *   packed (dev) [B,P_max,row_len] or NULL; unpacked (dev) [B,W,L,row_len] or NULL
 *   match_len (dev) [B,W]; best_beam, accept_len (dev) [B];
 *   accepted_tokens (dev) [B,L]
 * An unpacker entry of -1 (a padding candidate of a ragged batch) unpacks
 * to a zero row.
 */
int rd_unpack_accept(const int32_t *beams, const int32_t *unpacker,
                     const int32_t *packed_argmax, const void *packed, void *unpacked,
                     int dtype, int64_t row_len, int B, int W, int L,
                     int32_t *match_len, int32_t *best_beam, int32_t *accept_len,
                     int32_t *accepted_tokens, rd_stream_t stream);

/*
 * Steps 3b + 4 for a ragged batch (beam_width, beam_len as for
 * rd_pack_beams_mask_ragged).  Only beams w < beam_width[b] and positions
 * below beam_len[b] take part: n <= beam_len[b]-1, padding beams get
 * match_len -1, and a request with no beam or no position accepts nothing
 * (best_beam = accept_len = -1, accepted_tokens all -1, which
 * rd_commit_accepted leaves unchanged).  Padding candidates unpack to zero
 * rows.  Otherwise exactly rd_unpack_accept.
 */
int rd_unpack_accept_ragged(const int32_t *beams, const int32_t *beam_width,
                            const int32_t *beam_len, const int32_t *unpacker,
                            const int32_t *packed_argmax, const void *packed, void *unpacked,
                            int dtype, int64_t row_len, int B, int W, int L,
                            int32_t *match_len, int32_t *best_beam, int32_t *accept_len,
                            int32_t *accepted_tokens, rd_stream_t stream);

/*
 * Step 4, stochastic variant: multi-step speculative sampling over the
 * token tree.  [SURV] rejection sampling: a draft x ~ q kept when
 * u < p(x)/q(x) is distributed as p; [SURV] SpecInfer: random decoding
 * tests each drafted candidate in turn and, when all are rejected, samples
 * what remains of p, matching the target's sampling distribution.
 * Walk from slot 0 (beam 0's depth-0 node).  At node u, p = softmax of
 * logits[b,u,:] (fp32) and q = q[b,u,:] (the drafter's distribution for the
 * next token).  Children of u are tried in increasing slot order; the i-th
 * tried at depth d, token x = packed_tokens[b,child], is accepted when
 * u_accept[b,d,i] * q(x) < p(x), and the walk moves to it; a rejection
 * replaces p by max(p - q, 0) / sum (p kept if the sum is 0).  When no child
 * is accepted or u is a leaf, the bonus token is the first index whose
 * running sum of p exceeds u_bonus[b] times its total.
 *
 *   unpacker, packed_len, packed_tokens (dev) from rd_pack_beams*
 *   logits (dev) [B,P_max,V] in dtype (e.g. rd_lm_head_argmax's output)
 *   q (dev) fp32 [B,P_max,V]; u_accept (dev) fp32 [B,L,W]; u_bonus (dev) fp32 [B]
 *   best_beam, accept_len (dev) [B]: the lowest beam holding the last
 *     accepted node and the number n of accepted drafts (-1 for an empty
 *     request), as rd_unpack_accept reports them for rd_commit_accepted
 *   accepted_tokens (dev) [B,L]: n drafts, then the bonus, then -1
 *   path (dev) [B,L] or NULL: slots of the walk from depth 0, then -1
 *   ws (dev) workspace >= rd_stochastic_accept_workspace_size(B, W, L)
 *           (12 bytes a slot): per slot, the two values of its own test at
 *           its parent and the bonus token it yields if all its children
 *           are rejected
 * Two launches (every slot's statistics, then one walk per request);
 * deterministic.  Errors: RD_E_ARG for null required pointers or negative
 * sizes, RD_E_UNSUPPORTED for W > 64, L > 16 or an unknown dtype,
 * RD_E_WORKSPACE for a small workspace.
 */
size_t rd_stochastic_accept_workspace_size(int B, int W, int L);
int rd_stochastic_accept(int dtype, const int32_t *unpacker, const int32_t *packed_len,
                         const int32_t *packed_tokens, const void *logits, const float *q,
                         const float *u_accept, const float *u_bonus, int B, int W, int L, int V,
                         int32_t *best_beam, int32_t *accept_len, int32_t *accepted_tokens,
                         int32_t *path, void *ws, size_t ws_bytes, rd_stream_t stream);

/*
 * After step 4 -- commit the accepted path.  [TRT] intro: the best path is
 * accepted before the next drafting round, so its tokens join the context;
 * [NEWS] "RNN draft model": the drafter continues from the target's latest
 * token and the target's last hidden state.
 * For request b with w = best_beam[b], n = accept_len[b], c = kv_len[b]
 * (as rd_unpack_accept leaves them): candidates (b,w,0..n) -- the initial
 * token and the n accepted drafts -- were verified over exactly their plain
 * decoding context, so for j = 0..n and every KV head g
 *   k_cache[b,g,c+j,:] = k_new[b, unpacker[b,w,j], g, :]   (v likewise),
 * then kv_len[b] = c + n + 1, and, when hidden and hidden_next are given,
 *   hidden_next[b,:] = hidden[b, unpacker[b,w,n], :]
 * (the row whose logits chose the bonus token).  The bonus token itself has
 * no key or value yet: it opens the next step's beams.
 * A request with w outside [0,W), n outside [0,L-1], c < 0 or c+n+1 > S_max
 * is left unchanged (cache rows, kv_len and its hidden_next row), so a
 * caller sees an overflow as kv_len not moving.  Unpacker entries are
 * clamped to [0, W*L).
 *
 *   unpacker (dev) [B,W,L]; best_beam, accept_len (dev) [B]
 *   k_new, v_new (dev) [B,W*L,Hkv,D] in dtype (packed layout, read only)
 *   hidden (dev) [B,W*L,K] or NULL; hidden_next (dev) [B,K] or NULL (both or neither)
 *   k_cache, v_cache (dev) [B,Hkv,S_max,D] in dtype, updated in place
 *   kv_len (dev) [B], read and advanced in place
 * One launch.  The written cache rows must not overlap k_new, v_new or
 * hidden.  Errors: RD_E_ARG for null required pointers, negative sizes,
 * Hkv < 1, D < 1, or only one of hidden / hidden_next given;
 * RD_E_UNSUPPORTED for W > 64, L > 16, an unknown dtype, or one request's
 * rows exceeding 2^31 bytes.
 */
int rd_commit_accepted(int dtype, const int32_t *unpacker, const int32_t *best_beam,
                       const int32_t *accept_len, const void *k_new, const void *v_new,
                       const void *hidden, int B, int W, int L, int Hkv, int D, int K,
                       int S_max, void *k_cache, void *v_cache, int32_t *kv_len,
                       void *hidden_next, rd_stream_t stream);

/*
 * rd_commit_accepted into a paged cache (pools and block table as for
 * rd_tree_attention_paged): logical position t = kv_len[b] + j goes to row
 * t % page_size of page block_table[b, t / page_size]; the capacity is
 * max_pages * page_size.  The caller gives every request table entries for
 * the positions it may commit.  A request whose committed positions reach a
 * table entry outside [0, num_pages) (e.g. -1 for "no page yet") is left
 * unchanged, like an overflow: its kv_len does not move and no page is
 * written, so a commit never writes into a page it was not given.
 * Same rows, hidden state, overflow rule, launch count and errors as
 * rd_commit_accepted, plus RD_E_ARG for page_size < 1, negative num_pages
 * or max_pages, or a null pool or table.
 *
 *   k_pages, v_pages (dev) [num_pages, Hkv, page_size, D] in dtype, updated in place
 *   block_table (dev) int32 [B, max_pages]
 */
int rd_commit_accepted_paged(int dtype, const int32_t *unpacker, const int32_t *best_beam,
                             const int32_t *accept_len, const void *k_new, const void *v_new,
                             const void *hidden, int B, int W, int L, int Hkv, int D, int K,
                             void *k_pages, void *v_pages, int64_t num_pages, int page_size,
                             const int32_t *block_table, int max_pages, int32_t *kv_len,
                             void *hidden_next, rd_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RD_H */
