"""Choice of the tokens a full-size GPU test checks against the oracle. Host-side bookkeeping only:
nothing here computes any part of the MoE layer."""
import numpy as np

TILE_HEIGHTS = (128, 192, 256)  # every M-tile height the grouped GEMMs take


def cover_tokens(offsets, perm, inv, k, n_min, seed, heights=TILE_HEIGHTS):
    """Tokens whose routed rows hit every M tile [off_e + i*bm, min(off_e + (i+1)*bm, off_{e+1}))
    of every expert e for every tile height bm, and every expert's first and last row; then random
    tokens until there are n_min (or every token). A tile that an already chosen token's rows hit
    is skipped (greedy cover). offsets, perm, inv: the schedule (inv = -1 for a dropped
    assignment). Returns the sorted token ids."""
    offsets = np.asarray(offsets, np.int64)
    perm = np.asarray(perm, np.int64)
    inv = np.asarray(inv, np.int64)
    R = int(offsets[-1])
    T = inv.size // k
    rng = np.random.default_rng(seed)
    hit = np.zeros(R, bool)
    seen = set()

    def add(t):
        if t in seen:
            return
        seen.add(t)
        rows = inv[t * k:(t + 1) * k]
        hit[rows[rows >= 0]] = True

    E = offsets.size - 1
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            add(int(perm[a]) // k)
            add(int(perm[b - 1]) // k)
    for bm in heights:
        for e in range(E):
            a, b = int(offsets[e]), int(offsets[e + 1])
            for r0 in range(a, b, bm):
                r1 = min(b, r0 + bm)
                if not hit[r0:r1].any():
                    add(int(perm[int(rng.integers(r0, r1))]) // k)
    while len(seen) < min(n_min, T):
        add(int(rng.integers(0, T)))
    return np.array(sorted(seen), np.int64)
