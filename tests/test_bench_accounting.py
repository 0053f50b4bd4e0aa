"""The benchmark's count of computed work, pinned to its closed form.

For queries in natural order, query block i of a segment sees exactly the segment's keys with
original position <= its last row: (i - s*bps + 1) * Bs of them, whatever the permutation inside
the segment.  The bench counts the attention kernel's own-segment work from the live `perm`
(visible keys per query block, rounded up to 32-key stages, in units of Bs keys); on any valid
per-segment permutation that must equal the natural-order triangle.  A "permutation" that
repeats a position must change the count."""
import numpy as np

import bench


def _perm(B, H, N, S, seed):
    rng = np.random.default_rng(seed)
    p = np.empty((B, H, N), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for s0 in range(0, N, S):
                p[b, h, s0:s0 + S] = s0 + rng.permutation(S)
    return p


def test_own_segment_work_is_the_causal_triangle():
    for (B, H, N, S, Bs, G) in [(1, 2, 4096, 1024, 128, 4), (2, 1, 1536, 512, 64, 3),
                                (1, 3, 8192, 8192, 128, 1)]:
        perm = _perm(B, H, N, S, seed=N + S)
        bps = S // Bs
        tri = sum(i % bps + 1 for i in range(N // Bs))
        assert bench.own_segment_blocks(perm, Bs, S, G) == B * H * G * tri


def test_own_segment_work_sees_a_broken_permutation():
    B, H, N, S, Bs, G = 1, 1, 2048, 1024, 128, 1
    perm = _perm(B, H, N, S, seed=5)
    bps = S // Bs
    tri = sum(i % bps + 1 for i in range(N // Bs))
    bad = perm.copy()
    late = int(np.argmax(bad[0, 0, :S]))         # the key at position S-1 ...
    bad[0, 0, late] = 0                            # ... now repeats position 0: seen too early
    assert bench.own_segment_blocks(bad, Bs, S, G) != tri


def test_diagonal_skip_count_brute_force():
    """The diagonal tiles the attention kernel skips: a 32-row wave tile and a 32-key stage of a
    query block's own Bs positions are skipped when no (row, key) pair in them is causal-visible.
    Counted element by element on every tile of one Bs x Bs diagonal block."""
    for Bs in (64, 128):
        rows = np.arange(Bs)
        visible = rows[:, None] >= rows[None, :]          # key position <= row position
        W = Bs // 32
        skipped = sum(1 for w in range(W) for s in range(W)
                      if not visible[w * 32:(w + 1) * 32, s * 32:(s + 1) * 32].any())
        per_block = skipped / (W * W)                     # block-equivalents per query block
        B, Hq, nb = 2, 3, 5
        assert bench.diag_skipped_blocks(B, Hq, nb, Bs) == B * Hq * nb * per_block
