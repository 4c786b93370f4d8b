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
