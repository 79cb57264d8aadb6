"""Independent statement of the work partition the host planner must produce.

Test infrastructure only (see the package docstring).

The pages fix *that* the key axis is split (split-K / split-KV, [Triton-hd512] section
"Not covered"; [VO-split] section "NVFP4 split-KV correctness (added)"), not how.  The
result of attention does not depend on the partition (merge of any partition equals the
unsplit result, which the oracle tests pin), so this module is not part of what attention
computes: it restates, in plain Python, the partition rule the C planner documents, so the
planner's integer output can be compared with it exactly.

Decode rule (units of 16-token logical blocks, block j = tokens [16j, 16j+16)):

* L_b from the page table; visible keys are [s_b, L_b) with s_b = max(0, L_b - W) when a
  window W > 0 is set, else 0.
* Visible blocks: fb = s_b // 16, eb = ceil(L_b / 16), n_b = eb - fb.
* Number of chunks: fixed ``num_splits`` S > 0 gives c_b = min(S, n_b); adaptive (S = 0)
  uses ``chunk_blocks = max(MIN_CHUNK_BLOCKS, ceil(sum_b n_b / ceil(TARGET_WGS / Hkv)))``
  and c_b = min(MAX_SPLITS, ceil(n_b / chunk_blocks)).  c_b is at least 1.
* Chunk c of request b spans blocks [fb + n_b*c // c_b, fb + n_b*(c+1) // c_b), clipped to
  the visible keys.
* Requests with c_b > 1 own c_b consecutive workspace slots, in request order; a request
  with a single chunk writes its output directly (slot -1).
* Work items run longest first (token count descending), ties in (b, c) order.

Prefill rule: the query rows of one (request, KV head) are the q_len * G pairs
(token i, head g) flattened as i * G + g; tiles of ``tile_rows`` consecutive rows;
a tile sees keys [kv_begin, kv_end) with kv_end = pos(last token) + 1 under the causal
mask (L_b without it) and kv_begin = max(0, pos(first token) - W + 1) with a window.
Tiles run by key count descending, ties in (b, tile) order.
"""

BLOCK_TOKENS = 16
TARGET_WGS = 2048
MIN_CHUNK_BLOCKS = 8
MAX_SPLITS = 64


def _ceil_div(a, b):
    return -(-a // b)


def decode_partition_ref(kv_lens, window, num_splits, num_kv_heads):
    """Returns (items, merges).

    items:  list of (b, t_begin, t_end, slot) in execution order.
    merges: list of (b, slot_begin, num_chunks) for requests split into several chunks.
    """
    starts, nblk = [], []
    for length in kv_lens:
        length = int(length)
        s = max(0, length - window) if window > 0 else 0
        fb = s // BLOCK_TOKENS
        eb = _ceil_div(length, BLOCK_TOKENS)
        starts.append(s)
        nblk.append(max(0, eb - fb))
    if num_splits > 0:
        chunks = [max(1, min(num_splits, n)) for n in nblk]
    else:
        target_chunks = _ceil_div(TARGET_WGS, num_kv_heads)
        chunk_blocks = max(MIN_CHUNK_BLOCKS, _ceil_div(sum(nblk), target_chunks))
        chunks = [max(1, min(MAX_SPLITS, _ceil_div(n, chunk_blocks))) for n in nblk]

    items, merges, next_slot = [], [], 0
    for b, length in enumerate(kv_lens):
        length = int(length)
        c_b, n_b, s_b = chunks[b], nblk[b], starts[b]
        fb = s_b // BLOCK_TOKENS
        slot0 = -1
        if c_b > 1:
            slot0 = next_slot
            merges.append((b, next_slot, c_b))
            next_slot += c_b
        for c in range(c_b):
            lo = fb + (n_b * c) // c_b
            hi = fb + (n_b * (c + 1)) // c_b
            t0 = max(s_b, lo * BLOCK_TOKENS)
            t1 = min(length, hi * BLOCK_TOKENS)
            if length == 0:
                t0 = t1 = 0
            items.append((b, t0, t1, -1 if c_b == 1 else slot0 + c, c))
    items.sort(key=lambda it: (-(it[2] - it[1]), it[0], it[4]))
    return [it[:4] for it in items], merges


def prefill_tiles_ref(qo_lens, kv_lens, group, tile_rows, causal, window):
    """Returns the list of (b, row_begin, row_end, kv_begin, kv_end) in execution order."""
    tiles = []
    for b, (q_len, length) in enumerate(zip(qo_lens, kv_lens)):
        q_len, length = int(q_len), int(length)
        rows = q_len * group
        for j, r0 in enumerate(range(0, rows, tile_rows)):
            r1 = min(rows, r0 + tile_rows)
            pos_first = length - q_len + r0 // group
            pos_last = length - q_len + (r1 - 1) // group
            kv_end = pos_last + 1 if causal else length
            kv_begin = max(0, pos_first - window + 1) if window > 0 else 0
            tiles.append((b, r0, r1, kv_begin, kv_end, j))
    tiles.sort(key=lambda t: (-(t[4] - t[3]), t[0], t[5]))
    return [t[:5] for t in tiles]
