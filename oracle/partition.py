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
* Visible blocks: fb = s_b // 16, eb = ceil(L_b / 16), n_b = max(0, eb - fb).
* Work units are the (request b, KV head h, block j) triples, flattened in (b, h, j)
  order; the range of (b, h) is [o_bh, o_bh + n_b) and U is the total.
* Pieces (one wave each) cut the flattened axis into P near-equal parts
  [U p // P, U (p+1) // P): with P0 = min(WAVE_SLOTS, ceil(U / MIN_PIECE_BLOCKS)) and the
  largest part size m = ceil(U / P0), P = ceil(U / m), the fewest parts of at most m units.
  Pair-aligned instead, when S = 0 (no fixed split) and sum over (b, h) of
  c_bh = ceil(n_b / m) is at most WAVE_SLOTS: each (b, h) range on its own in c_bh
  near-equal parts [o_bh + n_b k // c_bh, o_bh + n_b (k+1) // c_bh), in (b, h) order.
* A fixed split S > 0 (split-K S) cuts every (b, h) range into c = min(S, n_b) chunks
  [o_bh + n_b k // c, o_bh + n_b (k+1) // c); S = 0 adds no cuts.
* A piece is cut at (b, h) boundaries and at chunk boundaries into segments, so every
  chunk is computed by one or more whole segments; blocks [j0, j1) of (b, h) cover the
  keys [max(s_b, 16 (fb + j0)), min(L_b, 16 (fb + j1))).
* Waves run by piece length descending, ties in piece order; consecutive runs of
  WAVES_PER_GROUP waves form workgroups.
* Grouping (when the kernel holds split results in LDS): the last segments of a run of two
  or more consecutive waves of one workgroup that belong to one (b, h) with several
  segments form a group, whose results are combined into one slot.
* A (b, h) with several segments owns one consecutive workspace slot per segment (one per
  group for grouped segments), in piece order, slots numbered in (b, h) order, and gets a
  merge entry (b, h, first slot, count); a (b, h) with one segment writes its output
  directly (slot -1); an empty request gets a merge entry with no slots for each h (zero
  output, lse -inf).

Prefill rule: the query rows of one (request, KV head) are the q_len * G pairs
(token i, head g) flattened as i * G + g; tiles of ``tile_rows`` consecutive rows;
a tile sees keys [kv_begin, kv_end) with kv_end = pos(last token) + 1 under the causal
mask (L_b without it) and kv_begin = max(0, pos(first token) - W + 1) with a window.
Split-K (a short query over a long KV; the split-KV geometry of [VO-split] section "NVFP4
split-KV correctness (added)"): a tile's stages are the 32-key blocks it touches,
S = ceil(kv_end / 32) - kv_begin // 32.  When tiles x H_kv < SPLIT_ITEMS, with
C = max(MIN_CHUNK_STAGES, ceil(total S x H_kv / SPLIT_ITEMS)), every tile with S > C is cut
into c = ceil(S / C) chunks covering keys [max(kv_begin, 32 (s0 + S k // c)),
min(kv_end, 32 (s0 + S (k+1) // c))), s0 = kv_begin // 32; chunks take consecutive
partial slots in (b, tile, chunk) order and the tile a merge entry (b, row_begin, row_end,
q_begin, first slot, c).  Items run by key count descending, ties in (b, tile, chunk)
order; except, without split-K, when the K and V bytes the tiles read (per request, the keys
from its tiles' smallest kv_begin to its largest kv_end, times H_kv times the bytes a key
takes in one KV head) exceed LAST_LEVEL_CACHE_BYTES: then request by request (requests in
the order of their longest tile in the first ordering, ties by b), key count descending
within each, so the tiles running together read one request's keys.
"""

BLOCK_TOKENS = 16
WAVE_SLOTS = 2048
WAVES_PER_GROUP = 8
MIN_PIECE_BLOCKS = 8
MAX_SPLITS = 64
PREFILL_STAGE = 32
LAST_LEVEL_CACHE_BYTES = 256 << 20  # the GPU's last-level (memory-side) cache
SPLIT_ITEMS = 512
MIN_CHUNK_STAGES = 8


def _ceil_div(a, b):
    return -(-a // b)


def decode_partition_ref(kv_lens, window, num_splits, num_kv_heads, group_last=False):
    """Returns (waves, merges, groups).

    waves:  in launch order, each a list of segments (b, h, t_begin, t_end, slot).
    merges: (b, h, slot_begin, num_slots) for every (request, KV head) that has several
            segments or no keys at all, in (b, h) order.
    groups: per wave in launch order, (size, first wave of the group within its
            workgroup) when its last segment is grouped, else (0, 0).
    """
    lens = [int(x) for x in kv_lens]
    starts, nblk = [], []
    for length in lens:
        s = max(0, length - window) if window > 0 else 0
        starts.append(s)
        nblk.append(max(0, _ceil_div(length, BLOCK_TOKENS) - s // BLOCK_TOKENS))
    pairs = [(b, h) for b in range(len(lens)) for h in range(num_kv_heads)]
    origin, total = [], 0
    for b, h in pairs:
        origin.append(total)
        total += nblk[b]

    p0 = min(WAVE_SLOTS, _ceil_div(total, MIN_PIECE_BLOCKS))
    m = _ceil_div(total, p0) if p0 > 0 else 0
    p = _ceil_div(total, m) if m > 0 else 0
    per_pair = [_ceil_div(nblk[b], m) if m > 0 else 0 for b, _ in pairs]
    if num_splits == 0 and m > 0 and sum(per_pair) <= WAVE_SLOTS:
        pieces = [(origin[i] + nblk[b] * k // c, origin[i] + nblk[b] * (k + 1) // c)
                  for i, ((b, _), c) in enumerate(zip(pairs, per_pair)) for k in range(c)]
    else:
        pieces = [(total * k // p, total * (k + 1) // p) for k in range(p)]

    def cuts_of(i):  # unit positions that end a segment inside pair i's range
        b = pairs[i][0]
        n = nblk[b]
        ends = {origin[i] + n}
        if num_splits > 0 and n > 0:
            c = min(num_splits, n)
            ends |= {origin[i] + n * k // c for k in range(1, c)}
        return sorted(ends)

    def pair_of(u):  # the (b, h) whose range holds flattened unit u (empty ranges hold none)
        for i in range(len(pairs)):
            if origin[i] <= u < origin[i] + nblk[pairs[i][0]]:
                return i
        raise AssertionError(u)

    piece_segs = []
    for u0, u1 in pieces:
        segs, u = [], u0
        while u < u1:
            i = pair_of(u)
            b, h = pairs[i]
            e = min([u1] + [x for x in cuts_of(i) if x > u])
            fb = starts[b] // BLOCK_TOKENS
            t0 = max(starts[b], (fb + u - origin[i]) * BLOCK_TOKENS)
            t1 = min(lens[b], (fb + e - origin[i]) * BLOCK_TOKENS)
            segs.append([b, h, t0, t1, -1])
            u = e
        piece_segs.append(segs)

    count = {}
    for segs in piece_segs:
        for sg in segs:
            count[(sg[0], sg[1])] = count.get((sg[0], sg[1]), 0) + 1
    order = sorted(range(len(pieces)), key=lambda k: (-(pieces[k][1] - pieces[k][0]), k))

    # Groups: runs of consecutive waves (launch order) inside one workgroup whose last
    # segments belong to the same split (b, h).
    lead, gsize, gpos = {}, {}, {}
    if group_last:
        last_key = [tuple(piece_segs[k][-1][:2]) for k in order]
        s = 0
        while s < len(order):
            e = s + 1
            if count[last_key[s]] > 1:
                while (e < len(order) and e // WAVES_PER_GROUP == s // WAVES_PER_GROUP
                       and last_key[e] == last_key[s]):
                    e += 1
            if e - s >= 2:
                for t in range(s, e):
                    lead[order[t]] = order[s]
                    gsize[order[t]] = e - s
                    gpos[order[t]] = s % WAVES_PER_GROUP
            s = e

    def grouped(k, j):
        return j == len(piece_segs[k]) - 1 and k in lead

    units = {}
    for k, segs in enumerate(piece_segs):
        for j, sg in enumerate(segs):
            key = (sg[0], sg[1])
            if count[key] > 1 and (not grouped(k, j) or lead[k] == k):
                units[key] = units.get(key, 0) + 1
    first_slot, merges, next_slot = {}, [], 0
    for b, h in pairs:
        k = count.get((b, h), 0)
        if k == 0:
            merges.append((b, h, next_slot, 0))
        elif k > 1:
            first_slot[(b, h)] = next_slot
            merges.append((b, h, next_slot, units[(b, h)]))
            next_slot += units[(b, h)]
    used, group_slot = {}, {}
    for k, segs in enumerate(piece_segs):
        for j, sg in enumerate(segs):
            key = (sg[0], sg[1])
            if key not in first_slot:
                continue
            if grouped(k, j) and lead[k] in group_slot:
                sg[4] = group_slot[lead[k]]
                continue
            sg[4] = first_slot[key] + used.get(key, 0)
            used[key] = used.get(key, 0) + 1
            if grouped(k, j):
                group_slot[lead[k]] = sg[4]

    waves = [[tuple(sg) for sg in piece_segs[k]] for k in order]
    groups = [(gsize[k], gpos[k]) if k in lead else (0, 0) for k in order]
    return waves, merges, groups


def prefill_plan_ref(qo_lens, kv_lens, group, tile_rows, causal, window, num_kv_heads,
                     kv_bytes_per_key=0):
    """Returns (items, merges).  kv_bytes_per_key: bytes of one key's K and V rows in one KV
    head (0: never order request by request).

    items:  in execution order, each (b, row_begin, row_end, kv_begin, kv_end, slot), slot
            -1 for a tile computed whole.
    merges: (b, row_begin, row_end, q_begin, slot_begin, num_slots) per split tile.
    """
    tiles, q_begin = [], 0
    for b, (q_len, length) in enumerate(zip(qo_lens, kv_lens)):
        q_len, length = int(q_len), int(length)
        rows = q_len * group
        for j, r0 in enumerate(range(0, rows, tile_rows)):
            r1 = min(rows, r0 + tile_rows)
            pos_first = length - q_len + r0 // group
            pos_last = length - q_len + (r1 - 1) // group
            kv_end = pos_last + 1 if causal else length
            kv_begin = max(0, pos_first - window + 1) if window > 0 else 0
            tiles.append((b, r0, r1, kv_begin, kv_end, q_begin))
        q_begin += q_len

    def stages(t):
        return _ceil_div(t[4], PREFILL_STAGE) - t[3] // PREFILL_STAGE if t[4] > t[3] else 0

    chunk = 0
    if len(tiles) * num_kv_heads < SPLIT_ITEMS:
        chunk = max(MIN_CHUNK_STAGES,
                    _ceil_div(sum(stages(t) for t in tiles) * num_kv_heads, SPLIT_ITEMS))
    items, merges, slots = [], [], 0
    for t in tiles:
        b, r0, r1, kb, ke, qb = t
        s = stages(t)
        if chunk == 0 or s <= chunk:
            items.append((b, r0, r1, kb, ke, -1))
            continue
        c = _ceil_div(s, chunk)
        merges.append((b, r0, r1, qb, slots, c))
        s0 = kb // PREFILL_STAGE
        for k in range(c):
            items.append((b, r0, r1, max(kb, PREFILL_STAGE * (s0 + s * k // c)),
                          min(ke, PREFILL_STAGE * (s0 + s * (k + 1) // c)), slots))
            slots += 1
    order = sorted(range(len(items)), key=lambda i: (-(items[i][4] - items[i][3]), i))
    span = {}
    for b, _, _, kb, ke, _ in items:
        lo, hi = span.get(b, (kb, ke))
        span[b] = (min(lo, kb), max(hi, ke))
    kv_bytes = sum(hi - lo for lo, hi in span.values()) * num_kv_heads * kv_bytes_per_key
    if chunk == 0 and kv_bytes > LAST_LEVEL_CACHE_BYTES:
        first = {}
        for i in order:
            first.setdefault(items[i][0], len(first))
        order = sorted(order, key=lambda i: first[items[i][0]])  # stable: lengths stay sorted
    return [items[i] for i in order], merges
