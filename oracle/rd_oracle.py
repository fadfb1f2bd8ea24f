"""CPU oracle for the ReDrafter verification step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct fp64 (numpy) statement of what one
verification step computes.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.
It shares no code with the HIP library and imports nothing from it.

Sources (cited by page title and section):
  [TRT] "ReDrafter in NVIDIA TensorRT-LLM" blog (Chinese and English copies),
        intro; "Inflight-batching Compatible Engine"; "Implementing in-Engine
        Validation and Drafting" (the PyTorch `unpack` listing).
  [NEWS] Apple/NVIDIA ReDrafter news article, sections "RNN draft model" and
        "Dynamic tree attention", and the greedy-decoding benchmark paragraph.
  [PAPER] "Recurrent Drafter for Fast Speculative Decoding in Large Language
        Models", abstract point (2).
  [SURV] "Accelerating LLM inference with speculative decoding" survey,
        section SpecInfer / "Token Tree Verifier".

Readings where the pages are silent (each listed with its reason in the
design notes): packed slots are in first-occurrence order of a beam-major
scan; beam position 0 is the target's initial token; attention scale is
1/sqrt(D) with every cached key visible; grouped-query heads map to KV head
h // (Hq/Hkv); argmax ties resolve to the lowest vocabulary id and equal
match lengths to the lowest beam index.

Pinned by tests that do not reuse this file's formulas: brute-force prefix
counting, exhaustive tiny beam sets, a PyTorch gather restating the pages'
unpack, PyTorch scaled-dot-product attention on single-beam trees, closed
forms (self-only attention, uniform scores, one-hot projections), GQA versus
repeated-head MHA, and hand-worked accept cases under tests/golden/.  The
commit of the accepted path is pinned by decoding over the committed cache
(torch scaled-dot-product attention must reproduce verification's output
for every accepted candidate), by the committed rows spelling the text that
the greedy accept reports, and by the chosen hidden state re-deriving the
bonus token.  Paged attention is pinned by pools cut from a contiguous cache
with numpy reshapes (identity page tables reproduce contiguous attention
exactly) and by invariance under permuting the pool's pages.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "pack_beams", "tree_mask", "mask_to_bits", "attention_per_beam",
    "attention_packed", "gather_pages", "attention_paged", "lm_head_logits", "argmax_first", "unpack",
    "greedy_accept", "stochastic_accept", "commit_accepted", "commit_accepted_paged", "verify_requests",
]


# ---------------------------------------------------------------- step 1 --
def pack_beams(beams: np.ndarray, beam_width=None, beam_len=None) -> dict:
    """Deduplicate shared prefixes of each request's beams with a literal trie.

    [NEWS] "Dynamic tree attention" and [PAPER] abstract (2): the beams that
    beam search returns share prefixes; the shared prefixes are found and
    removed from the tokens the target verifies.  [TRT] PyTorch `unpack`:
    the unpacker has shape [batch, beam_width, beam_length] and indexes
    dimension 1 of the packed tensor.

    A trie node is a distinct prefix beams[b, w, 0..l].  Nodes are numbered
    in the order a beam-major scan first meets them (trie insertion order),
    so a parent always precedes its children.

    Returns int32 arrays: tokens [B,P] (pad -1), length [B], unpacker
    [B,W,L], depth [B,P] (pad -1), src [B,P] = w*L+l of the first
    occurrence (pad -1), with P = W*L.

    Ragged batches ([TRT] "Inflight-batching Compatible Engine": requests in
    one batch differ).  Reading: request b has beam_width[b] <= W beams of
    beam_len[b] <= L tokens, stored in the top-left corner of its [W, L]
    slab; the rest is padding that opens no node and gets unpacker -1.
    """
    beams = np.asarray(beams)
    B, W, L = beams.shape
    bw = [W] * B if beam_width is None else [min(max(int(x), 0), W) for x in beam_width]
    bl = [L] * B if beam_len is None else [min(max(int(x), 0), L) for x in beam_len]
    P = W * L
    tokens = np.full((B, P), -1, np.int32)
    depth = np.full((B, P), -1, np.int32)
    src = np.full((B, P), -1, np.int32)
    length = np.zeros(B, np.int32)
    unpacker = np.full((B, W, L), -1, np.int32)
    for b in range(B):
        child = {}  # (parent node or -1 for the virtual root, token) -> node
        n = 0
        for w in range(bw[b]):
            cur = -1
            for l in range(bl[b]):
                key = (cur, int(beams[b, w, l]))
                if key not in child:
                    child[key] = n
                    tokens[b, n] = beams[b, w, l]
                    depth[b, n] = l
                    src[b, n] = w * L + l
                    n += 1
                cur = child[key]
                unpacker[b, w, l] = cur
        length[b] = n
    return {"tokens": tokens, "length": length, "unpacker": unpacker, "depth": depth, "src": src}


def tree_mask(unpacker: np.ndarray, packed_len: np.ndarray) -> np.ndarray:
    """Tree-causal mask, bool [B, P, P]: mask[b,p,q] iff q is p or an ancestor of p.

    [SURV] SpecInfer "Token Tree Verifier": the tree is laid out in a
    depth-first-compatible order and one topology-aware causal mask lets a
    single kernel evaluate every path.  Node p = unpacker[b,w,l] has as
    ancestors-or-self exactly the nodes unpacker[b,w,0..l] on its beam.
    Rows and columns at or beyond packed_len are zero; padding candidates
    (unpacker -1) are skipped.
    """
    B, W, L = unpacker.shape
    P = W * L
    mask = np.zeros((B, P, P), dtype=bool)
    for b in range(B):
        for w in range(W):
            for l in range(L):
                p = unpacker[b, w, l]
                if p < 0:
                    continue
                for j in range(l + 1):
                    mask[b, p, unpacker[b, w, j]] = True
        n = int(packed_len[b])
        mask[b, n:, :] = False
        mask[b, :, n:] = False
    return mask


def mask_to_bits(mask: np.ndarray) -> np.ndarray:
    """Bit-packed mask rows: uint32 [B, P, ceil(P/32)], bit (q % 32) of word q // 32."""
    B, P, _ = mask.shape
    nw = (P + 31) // 32
    out = np.zeros((B, P, nw), dtype=np.uint32)
    for q in range(P):
        out[:, :, q // 32] |= (mask[:, :, q].astype(np.uint32) << np.uint32(q % 32))
    return out


# ---------------------------------------------------------------- step 2 --
def _softmax_weighted_sum(scores: np.ndarray, values: np.ndarray) -> np.ndarray:
    """softmax over the last axis of `scores` [..., T] applied to values [..., T, D]."""
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    e /= e.sum(axis=-1, keepdims=True)
    return np.matmul(e[..., None, :], values)[..., 0, :]


def attention_per_beam(q, k, v, k_cache, v_cache, kv_len, scale=None) -> np.ndarray:
    """Causal attention of every candidate over its own beam alone (no dedup).

    [TRT] intro and FAQ: the target verifies draft tokens from several
    paths with tree-style attention; [NEWS] "Dynamic tree attention":
    removing shared prefixes only reduces the data processed, so the result
    must equal attending over each beam by itself.  This is that definition.

    q [B,W,L,Hq,D]; k, v [B,W,L,Hkv,D]; k_cache, v_cache [B,Hkv,S,D];
    kv_len [B].  For candidate (b,w,l) and head h with KV head
    g = h // (Hq/Hkv): keys are k_cache[b,g,0:kv_len[b]] followed by
    k[b,w,0..l,g]; scores are q.k * scale (default 1/sqrt(D)); softmax;
    weighted sum of the matching values.  Returns fp64 [B,W,L,Hq,D].
    """
    q = np.asarray(q, np.float64)
    B, W, L, Hq, D = q.shape
    Hkv = k.shape[3]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.zeros((B, W, L, Hq, D), np.float64)
    for b in range(B):
        n = int(kv_len[b])
        kc = np.asarray(k_cache[b, :, :n], np.float64)          # [Hkv, n, D]
        vc = np.asarray(v_cache[b, :, :n], np.float64)
        for w in range(W):
            kb = np.asarray(k[b, w], np.float64)                 # [L, Hkv, D]
            vb = np.asarray(v[b, w], np.float64)
            for l in range(L):
                qg = q[b, w, l].reshape(Hkv, G, D)               # head h = g*G + j
                s_cache = np.matmul(qg, kc.transpose(0, 2, 1))    # [Hkv, G, n]
                kn = kb[:l + 1].transpose(1, 0, 2)                # [Hkv, l+1, D]
                vn = vb[:l + 1].transpose(1, 0, 2)
                s_new = np.matmul(qg, kn.transpose(0, 2, 1))      # [Hkv, G, l+1]
                scores = np.concatenate([s_cache, s_new], axis=-1) * scale
                vals = np.concatenate([vc, vn], axis=1)           # [Hkv, n+l+1, D]
                o = np.stack([_softmax_weighted_sum(scores[g], vals[g]) for g in range(Hkv)])
                out[b, w, l] = o.reshape(Hq, D)
    return out


def attention_packed(q, k, v, k_cache, v_cache, kv_len, mask, packed_len, scale=None) -> np.ndarray:
    """Tree attention over packed tokens with the tree-causal mask.

    [SURV] "Token Tree Verifier": all paths in one pass under one mask.
    q [B,P,Hq,D]; k, v [B,P,Hkv,D]; mask bool [B,P,P].  Packed query p sees
    every cached key plus the packed keys q' with mask[b,p,q'].  Rows at or
    beyond packed_len are zero.  Returns fp64 [B,P,Hq,D].
    """
    q = np.asarray(q, np.float64)
    B, P, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.zeros((B, P, Hq, D), np.float64)
    for b in range(B):
        n = int(kv_len[b])
        kc = np.asarray(k_cache[b, :, :n], np.float64)
        vc = np.asarray(v_cache[b, :, :n], np.float64)
        for p in range(int(packed_len[b])):
            vis = np.nonzero(mask[b, p])[0]
            qg = q[b, p].reshape(Hkv, G, D)
            kn = np.asarray(k[b, vis], np.float64).transpose(1, 0, 2)   # [Hkv, nv, D]
            vn = np.asarray(v[b, vis], np.float64).transpose(1, 0, 2)
            scores = np.concatenate([np.matmul(qg, kc.transpose(0, 2, 1)),
                                     np.matmul(qg, kn.transpose(0, 2, 1))], axis=-1) * scale
            vals = np.concatenate([vc, vn], axis=1)
            o = np.stack([_softmax_weighted_sum(scores[g], vals[g]) for g in range(Hkv)])
            out[b, p] = o.reshape(Hq, D)
    return out


def gather_pages(pages: np.ndarray, block_table: np.ndarray, kv_len: np.ndarray) -> np.ndarray:
    """Logical KV cache of each request from a paged pool.

    [TRT] intro: the engine keeps its KV cache in pages (paged KV caching).
    Reading (the pages name the feature, not a layout): pages is
    [num_pages, Hkv, page_size, D]; key t of request b lives in page
    block_table[b, t // page_size] at slot t % page_size.  Only keys
    t < kv_len[b] are read (table entries past them may be anything).
    Returns [B, Hkv, max(kv_len), D] with zeros past each kv_len.
    """
    ps = pages.shape[2]
    B = block_table.shape[0]
    S = int(max(int(x) for x in kv_len)) if B else 0
    out = np.zeros((B, pages.shape[1], S, pages.shape[3]), pages.dtype)
    for b in range(B):
        for t in range(int(kv_len[b])):
            out[b, :, t] = pages[int(block_table[b, t // ps]), :, t % ps]
    return out


def attention_paged(q, k, v, k_pages, v_pages, block_table, kv_len, mask, packed_len, scale=None) -> np.ndarray:
    """Tree attention whose cached keys/values come from a paged pool.

    The plain definition: gather each request's logical cache from the pool
    (gather_pages), then attend exactly as attention_packed does.
    """
    kc = gather_pages(k_pages, block_table, kv_len)
    vc = gather_pages(v_pages, block_table, kv_len)
    return attention_packed(q, k, v, kc, vc, kv_len, mask, packed_len, scale)


# ---------------------------------------------------------------- step 3 --
def lm_head_logits(hidden: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """logits = hidden . weight^T in fp64; weight is [V, K] (nn.Linear layout).

    [NEWS] benchmark paragraph: verification is greedy decoding, so each
    candidate needs the target's logits over the vocabulary.
    """
    h = np.asarray(hidden, np.float64)
    w = np.asarray(weight, np.float64)
    return np.matmul(h, w.T)


def argmax_first(logits: np.ndarray) -> np.ndarray:
    """Index of the largest logit along the last axis; the lowest index wins ties."""
    return np.argmax(logits, axis=-1).astype(np.int32)


def unpack(packed: np.ndarray, unpacker: np.ndarray) -> np.ndarray:
    """[TRT] PyTorch `unpack`: out[b,w,l,:] = packed[b, unpacker[b,w,l], :].

    packed [B,P,X] (rank 3), unpacker [B,W,L] -> [B,W,L,X].  Padding
    candidates of ragged requests (unpacker -1) get zero rows.
    """
    packed = np.asarray(packed)
    assert packed.ndim == 3
    B, W, L = unpacker.shape
    out = np.zeros((B, W, L, packed.shape[2]), dtype=packed.dtype)
    for b in range(B):
        for w in range(W):
            for l in range(L):
                if unpacker[b, w, l] >= 0:
                    out[b, w, l] = packed[b, unpacker[b, w, l]]
    return out


# ---------------------------------------------------------------- step 4 --
def greedy_accept(beams: np.ndarray, target: np.ndarray, beam_width=None, beam_len=None) -> dict:
    """Greedy acceptance of the best beam plus one bonus token.

    [TRT] intro: tokens are verified and the best path is accepted before
    the next drafting round; [NEWS] greedy decoding; [NEWS] "RNN draft
    model": the drafter starts from the target's own initial token, so beam
    position 0 is that token and position j+1 is a draft that the target's
    prediction at position j must equal.

    target [B,W,L] = target argmax at every candidate position.  For beam
    w, n_w is the largest n <= L-1 with beams[b,w,j+1] == target[b,w,j] for
    all j < n.  The best beam is the lowest index with the largest n_w; the
    accepted tokens are beams[b,best,1..n] followed by the bonus
    target[b,best,n].

    Returns int32: match_len [B,W], best_beam [B], accept_len [B] (= n),
    accepted_tokens [B,L] (n drafts + bonus, pad -1).

    Ragged requests (see pack_beams): only beams w < beam_width[b] and
    positions below beam_len[b] take part; padding beams get match_len -1,
    and a request with no beam or no position accepts nothing (best_beam
    and accept_len -1, accepted_tokens all -1).
    """
    B, W, L = beams.shape
    bw = [W] * B if beam_width is None else [min(max(int(x), 0), W) for x in beam_width]
    bl = [L] * B if beam_len is None else [min(max(int(x), 0), L) for x in beam_len]
    match_len = np.full((B, W), -1, np.int32)
    best_beam = np.full(B, -1, np.int32)
    accept_len = np.full(B, -1, np.int32)
    accepted = np.full((B, L), -1, np.int32)
    for b in range(B):
        if bw[b] == 0 or bl[b] == 0:
            continue
        best, best_n = 0, -1
        for w in range(bw[b]):
            n = 0
            while n < bl[b] - 1 and beams[b, w, n + 1] == target[b, w, n]:
                n += 1
            match_len[b, w] = n
            if n > best_n:
                best, best_n = w, n
        best_beam[b] = best
        accept_len[b] = best_n
        toks = [int(t) for t in beams[b, best, 1:best_n + 1]] + [int(target[b, best, best_n])]
        accepted[b, :len(toks)] = toks
    return {"match_len": match_len, "best_beam": best_beam, "accept_len": accept_len,
            "accepted_tokens": accepted}


def _children(unpacker_b: np.ndarray, n: int) -> list:
    """Children of every slot of one request's tree, in increasing slot order."""
    W, L = unpacker_b.shape
    kids = [set() for _ in range(n)]
    for w in range(W):
        for l in range(L - 1):
            s, c = int(unpacker_b[w, l]), int(unpacker_b[w, l + 1])
            if 0 <= s < n and 0 <= c < n:
                kids[s].add(c)
    return [sorted(k) for k in kids]


def stochastic_accept(beams, unpacker, packed_len, packed_tokens, logits, q, u_accept, u_bonus) -> dict:
    """Stochastic verification of the token tree by multi-step speculative sampling.

    [SURV] "rejection sampling": with proposal q and target p, a sample x
    drawn from q and kept when u < p(x)/q(x), u ~ U(0,1), is distributed as
    p.  [SURV] SpecInfer: random decoding verifies the tree by multi-step
    speculative sampling -- each drafted candidate in turn gets that test;
    when every candidate is rejected, the sample comes from what is left of
    p -- and the result has the target's sampling distribution.

    Readings (the pages give the rule, not the tree walk): the walk starts at
    slot 0, the depth-0 node of beam 0 (the shared initial token).  At node
    u, p = softmax(logits[b, u]) and q = q[b, u] (the drafter's distribution
    for the token after u).  Children of u are tried in increasing slot
    order; the i-th child tried at depth d, token x, is accepted when
    u_accept[b, d, i] * q(x) < p(x), and the walk moves to it.  A rejection
    replaces p by max(p - q, 0) / sum(max(p - q, 0)) (q unchanged; if that
    sum is 0, p stays).  When no child is accepted, or u is a leaf, the bonus
    token is the smallest k with cumsum(p)[k] > u_bonus[b] * sum(p).

    logits, q [B,P,V]; u_accept [B,L,W]; u_bonus [B].  Returns int32:
    accept_len [B] (accepted drafts n), best_beam [B] (lowest beam whose
    depth-n node is the last accepted one), accepted_tokens [B,L] (the n
    drafts then the bonus, pad -1), path [B,L] (slots from depth 0, pad -1).
    """
    B, W, L = unpacker.shape
    accept_len = np.full(B, -1, np.int32)
    best_beam = np.full(B, -1, np.int32)
    accepted = np.full((B, L), -1, np.int32)
    path = np.full((B, L), -1, np.int32)
    for b in range(B):
        n_slots = int(packed_len[b])
        if n_slots == 0:
            continue
        kids = _children(unpacker[b], n_slots)
        u, d, toks = 0, 0, []
        path[b, 0] = 0
        while True:
            lg = np.asarray(logits[b, u], np.float64)
            e = np.exp(lg - lg.max())
            p = e / e.sum()
            qq = np.asarray(q[b, u], np.float64)
            moved = False
            for i, c in enumerate(kids[u]):
                x = int(packed_tokens[b, c])
                if u_accept[b, d, i] * qq[x] < p[x]:
                    u, d = c, d + 1
                    toks.append(x)
                    path[b, d] = c
                    moved = True
                    break
                res = np.maximum(p - qq, 0.0)
                z = res.sum()
                if z > 0:
                    p = res / z
            if not moved:
                break
        cdf = np.cumsum(p)
        bonus = int(np.searchsorted(cdf, u_bonus[b] * cdf[-1], side="right"))
        bonus = min(bonus, len(p) - 1)
        n = len(toks)
        accept_len[b] = n
        best_beam[b] = next(w for w in range(W) if unpacker[b, w, n] == u)
        accepted[b, :n + 1] = toks + [bonus]
    return {"accept_len": accept_len, "best_beam": best_beam, "accepted_tokens": accepted, "path": path}


# ------------------------------------------------------- after step 4 --
def commit_accepted(k, v, hidden, best_beam, accept_len, k_cache, v_cache, kv_len) -> dict:
    """Append the accepted path to the KV cache; pick the drafter's hidden state.

    [TRT] intro: the best path is accepted before the next drafting round,
    so its tokens join the context the next step attends to.  [NEWS] "RNN
    draft model": the drafter continues from the target's latest token and
    the target's last hidden state.

    Reading (the pages name the step, not its data movement): with
    w = best_beam[b] and n = accept_len[b], candidates (b,w,0..n) are the
    target's initial token and the n accepted drafts.  Their keys and values
    were computed during verification over exactly the context plain
    decoding gives them (the beam's own prefix plus the cache), so they are
    appended in order at positions kv_len[b] .. kv_len[b]+n of every KV head
    and kv_len[b] grows by n+1.  The bonus token has no key or value yet; it
    opens the next step's beams.  hidden_next[b] is the hidden state of
    candidate (b,w,n), whose logits chose the bonus token.  A request whose
    best_beam or accept_len is out of range, or whose appended rows would
    pass the cache capacity S, is left unchanged (committed[b] False,
    hidden_next[b] NaN): the pages say nothing about overflow.

    k, v [B,W,L,Hkv,D] and hidden [B,W,L,K] are per candidate (the unpacked
    definition); k_cache, v_cache [B,Hkv,S,D]; kv_len [B].  Returns fp64
    copies of the caches, int32 kv_len, bool committed [B], fp64
    hidden_next [B,K].
    """
    B, W, L = np.asarray(k).shape[:3]
    S = k_cache.shape[2]
    kc = np.array(k_cache, np.float64)
    vc = np.array(v_cache, np.float64)
    new_len = np.array(kv_len, np.int32)
    committed = np.zeros(B, bool)
    hidden_next = np.full((B, np.asarray(hidden).shape[3]), np.nan)
    for b in range(B):
        w, n, c = int(best_beam[b]), int(accept_len[b]), int(kv_len[b])
        if not (0 <= w < W and 0 <= n <= L - 1 and 0 <= c and c + n + 1 <= S):
            continue
        for j in range(n + 1):
            kc[b, :, c + j] = k[b, w, j]          # every KV head at once: [Hkv, D]
            vc[b, :, c + j] = v[b, w, j]
        new_len[b] = c + n + 1
        committed[b] = True
        hidden_next[b] = hidden[b, w, n]
    return {"k_cache": kc, "v_cache": vc, "kv_len": new_len, "committed": committed,
            "hidden_next": hidden_next}


def commit_accepted_paged(k, v, hidden, best_beam, accept_len, k_pages, v_pages, block_table, kv_len) -> dict:
    """commit_accepted into a paged cache (pools and table as in gather_pages).

    Logical position t of request b is row t % page_size of page
    block_table[b, t // page_size]; the capacity is max_pages * page_size.
    Same rows, same hidden state, same overflow rule as commit_accepted.
    A table entry that names no page of the pool (negative, or past the
    pool) gives its positions nowhere to go, so a request that would write
    one of them is treated like an overflow and left unchanged (the pages
    describe no paged layout at all; this is the reading that never writes
    a page the request does not own).
    """
    B, W, L = np.asarray(k).shape[:3]
    ps = k_pages.shape[2]
    num_pages = k_pages.shape[0]
    cap = block_table.shape[1] * ps
    kp = np.array(k_pages, np.float64)
    vp = np.array(v_pages, np.float64)
    new_len = np.array(kv_len, np.int32)
    committed = np.zeros(B, bool)
    hidden_next = np.full((B, np.asarray(hidden).shape[3]), np.nan)
    for b in range(B):
        w, n, c = int(best_beam[b]), int(accept_len[b]), int(kv_len[b])
        if not (0 <= w < W and 0 <= n <= L - 1 and 0 <= c and c + n + 1 <= cap):
            continue
        if not all(0 <= int(block_table[b, (c + j) // ps]) < num_pages for j in range(n + 1)):
            continue
        for j in range(n + 1):
            t = c + j
            page = int(block_table[b, t // ps])
            kp[page, :, t % ps] = k[b, w, j]
            vp[page, :, t % ps] = v[b, w, j]
        new_len[b] = c + n + 1
        committed[b] = True
        hidden_next[b] = hidden[b, w, n]
    return {"k_pages": kp, "v_pages": vp, "kv_len": new_len, "committed": committed,
            "hidden_next": hidden_next}


# ------------------------------------------------------------- the step --
def verify_requests(beams, q_unp, k_unp, v_unp, k_cache, v_cache, kv_len, hidden_unp, weight,
                    scale=None, want_logits=True) -> dict:
    """One verification step on a set of requests, in the unpacked definition.

    Everything is per candidate (b,w,l) with no deduplication except the
    pack/mask outputs, which are reported for comparison.  Arrays are
    indexed by position in the given set.
    """
    pk = pack_beams(beams)
    mask = tree_mask(pk["unpacker"], pk["length"])
    attn = attention_per_beam(q_unp, k_unp, v_unp, k_cache, v_cache, kv_len, scale)
    logits = lm_head_logits(hidden_unp, weight)
    target = argmax_first(logits)
    acc = greedy_accept(beams, target)
    out = {"pack": pk, "mask": mask, "mask_bits": mask_to_bits(mask), "attn": attn,
           "target": target, **acc}
    if want_logits:
        out["logits"] = logits
    return out
