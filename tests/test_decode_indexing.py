"""Host replay of the split-K kernels' block-table arithmetic (CPU only).

The compressed mainloop (decode_mainloop.hip) and the bypass mainloop
(decode_bypass.hip) read block-table entries before the sequence length is
known and dereference only some of them as page ids.  This replays, in plain
Python, which table index each wave dereferences for every (split, wave, chunk)
and checks over ragged lengths and split sizes that none lies at or past
ceil(T / 16): rows padded with anything (-1 included) past a sequence are safe.
"""

import itertools

import numpy as np

PAGE = 16
RING = 2  # chunks (compressed) or pages (bypass) held per wave


def ring_schedule(n):
    """Indices loaded by a wave with n items and a RING-deep register ring: the
    first RING loads, then one load per processed item, clamped to the last."""
    jmax = n - 1 if n > 0 else 0
    loads = [min(r, jmax) for r in range(RING)]
    j0 = 0
    while j0 + RING <= n:
        for r in range(RING):
            loads.append(min(j0 + r + RING, jmax))
        j0 += RING
    return loads


def compressed_pages(T, split_tokens, n_splits, max_blocks):
    """(table index or None for block 0) of every page the compressed mainloop loads."""
    out = []
    for split in range(n_splits):
        start = split * split_tokens
        if start >= T:
            continue
        end = min(T, start + split_tokens)
        for wave in range(4):
            span = end - start - 32 * wave
            nch = (span + 127) // 128 if span > 0 else 0
            # lane 2j + p of the wave's id vector: page p of chunk j
            lane_idx = [min((start + 32 * (wave + 4 * (ln >> 1)) + 16 * (ln & 1)) >> 4, max_blocks - 1)
                        for ln in range(64)]
            for j in ring_schedule(nch):
                c0 = start + 32 * (wave + 4 * j)
                if nch == 0:
                    out.append((None, None))  # both pages from block 0
                    continue
                b0 = lane_idx[2 * j]
                b1 = lane_idx[2 * j + 1] if c0 + 16 < end else b0
                out.append((b0, b1))
    return out


def bypass_pages(T, split_tokens, n_splits, max_blocks):
    out = []
    for split in range(n_splits):
        start = split * split_tokens
        if start >= T:
            continue
        end = min(T, start + split_tokens)
        npg = (end - start + PAGE - 1) // PAGE
        for wave in range(4):
            nj = (npg - wave + 3) >> 2 if npg > wave else 0
            if nj == 0:
                continue
            lane_idx = [min(start // PAGE + wave + 4 * ln, max_blocks - 1) for ln in range(64)]
            for j in ring_schedule(nj):
                out.append((lane_idx[j],))
    return out


def _cases():
    rng = np.random.default_rng(17)
    lens = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257, 1000, 4095, 4096, 4097, 20000]
    lens += [int(x) for x in rng.integers(1, 40000, 30)]
    for T in lens:
        for split_tokens in (64, 128, 256, 448, 1024, 2048, 4096):
            max_blocks = (T + PAGE - 1) // PAGE + int(rng.integers(0, 5))
            n_splits = (T + split_tokens - 1) // split_tokens + int(rng.integers(0, 3))
            yield T, split_tokens, n_splits, max_blocks


def test_compressed_mainloop_never_uses_padding_entries():
    for T, st, ns, mb in _cases():
        limit = (T + PAGE - 1) // PAGE
        for pair in compressed_pages(T, st, ns, mb):
            for idx in pair:
                assert idx is None or 0 <= idx < limit, (T, st, ns, mb, pair)


def test_bypass_mainloop_never_uses_padding_entries():
    for T, st, ns, mb in _cases():
        limit = (T + PAGE - 1) // PAGE
        for (idx,) in bypass_pages(T, st, ns, mb):
            assert 0 <= idx < limit, (T, st, ns, mb, idx)


def test_every_page_of_the_context_is_loaded():
    """The same replay covers the context: every page below ceil(T/16) is loaded
    by some wave (so the guards drop nothing that is needed)."""
    for T, st in itertools.product([1, 17, 100, 1000, 4097, 9000], [64, 256, 4096]):
        ns = (T + st - 1) // st
        limit = (T + PAGE - 1) // PAGE
        seen = {i for pair in compressed_pages(T, st, ns, limit) for i in pair if i is not None}
        assert seen == set(range(limit)), (T, st)
        seen_b = {i for (i,) in bypass_pages(T, st, ns, limit)}
        assert seen_b == set(range(limit)), (T, st)


# ---------------------------------------------------------------- item order
# Replay of split_items.hpp: a wave of 64 lanes, four sequences per lane and
# pass, an inclusive prefix sum over lanes, a ballot for the first lane whose
# running count passes the key.

def split_item(seq_lens, batch, Hkv, split_tokens, n_splits, work_list, wid):
    g, p = wid % Hkv, wid // Hkv
    if not work_list:
        return p // n_splits, p % n_splits, g
    per, span = 4, 256
    cap = n_splits * split_tokens

    def counts(base):
        whole, last = np.zeros((64, per), np.int64), np.zeros((64, per), np.int64)
        for lane in range(64):
            for k in range(per):
                i = base + per * lane + k
                t0 = int(seq_lens[i]) if i < batch else 0
                t = 0 if t0 <= 0 else min(t0, cap)
                whole[lane, k] = t // split_tokens
                last[lane, k] = int(t % split_tokens != 0)
        return whole, last

    n_whole = 0
    for base in range(0, batch, span):
        whole, last = counts(base)
        n_whole += int(np.cumsum(whole.sum(1))[63])
    in_whole = p < n_whole
    key = p if in_whole else p - n_whole
    carry = 0
    for base in range(0, batch, span):
        whole, last = counts(base)
        v = whole if in_whole else last
        own = v.sum(1)
        incl = np.cumsum(own)
        tot = int(incl[63])
        if key < carry + tot:
            lane = int(np.flatnonzero(carry + incl > key)[0])
            acc = carry + int(incl[lane]) - int(own[lane])
            for k in range(per):
                if key < acc + v[lane, k]:
                    return base + per * lane + k, (key - acc) if in_whole else int(whole[lane, k]), g
                acc += int(v[lane, k])
        carry += tot
    return -1, 0, g


def _live(seq_lens, Hkv, split_tokens, n_splits):
    cap = n_splits * split_tokens
    out = set()
    for b, t in enumerate(seq_lens):
        t = 0 if t <= 0 else min(int(t), cap)
        for s in range((t + split_tokens - 1) // split_tokens):
            out |= {(b, s, g) for g in range(Hkv)}
    return out


def test_work_list_covers_every_live_item_once_whole_splits_first():
    rng = np.random.default_rng(23)
    cases = []
    for batch in (1, 3, 64, 255, 256, 257, 600):
        lens = rng.integers(0, 5000, batch)
        lens[rng.random(batch) < 0.1] = 0
        cases.append((lens, 8 if batch < 300 else 2, 1024))
    special = np.array([0, 1, 1024, 1025, 2048, 4096 * 3, -5, 2 ** 31 - 1], np.int64)
    cases.append((special, 4, 4096))  # negative and far past max_seq_len: clamped
    for lens, Hkv, S in cases:
        n_splits = max(1, (int(max(0, min(lens.max(), 5000))) + S - 1) // S)
        grid = len(lens) * Hkv * n_splits
        got = [split_item(lens, len(lens), Hkv, S, n_splits, True, w) for w in range(grid)]
        live = [x for x in got if x[0] >= 0]
        assert len(live) == len(set(live)) and set(live) == _live(lens, Hkv, S, n_splits)
        # dense at the front, head fastest
        assert all(x[0] >= 0 for x in got[:len(live)]) and all(x[0] < 0 for x in got[len(live):])
        assert [x[2] for x in got[:len(live)]] == [w % Hkv for w in range(len(live))]
        # the whole splits come before every shorter last split
        cap = n_splits * S
        short = [min(max(int(lens[b]), 0), cap) < (s + 1) * S for b, s, g in live]
        assert short == sorted(short)
        assert all(0 <= s < n_splits for b, s, g in live)


def test_plain_order_is_a_bijection():
    for batch, Hkv, n_splits in ((16, 8, 4), (1, 8, 64), (5, 3, 7)):
        got = [split_item(None, batch, Hkv, 64, n_splits, False, w) for w in range(batch * Hkv * n_splits)]
        assert sorted(got) == sorted((b, s, g) for b in range(batch) for s in range(n_splits) for g in range(Hkv))
        assert [x[2] for x in got] == [w % Hkv for w in range(len(got))]
