"""CPU models of two pieces of the prefill kernel's index arithmetic.

Both are restated here from prefill_bf16.hip (the same integer formulas) so
that their invariants can be checked exhaustively on the host; the GPU parity
tests then exercise the kernel itself on shapes that reach each branch.

* Work-item numbering: (KV-head pair, query-tile rank, query head) from the
  work-group id, with pairs grouped across an XCD's share when a pair has
  fewer items than an XCD has CUs. It must be a bijection.
* Slot schedule with a window and initial-token anchors: the slots a wave
  visits (its anchor slots, then its own window up to its causal limit) must
  cover every key tile that holds a key visible to one of its rows.
"""
import pytest

CUS_PER_XCD = 32


def work_item(w, B, Hkv, n_qtiles, g):
    per_pair = n_qtiles * g
    n_pairs = B * Hkv
    total = n_pairs * per_pair
    G = 1 if per_pair >= CUS_PER_XCD else max(1, min(n_pairs, (total >> 3) // per_pair))
    grp = w // (G * per_pair)
    r_in = w - grp * G * per_pair
    row_items = min(G, n_pairs - grp * G) * g
    qrank = r_in // row_items
    rest = r_in - qrank * row_items
    return grp * G + rest // g, n_qtiles - 1 - qrank, rest % g


@pytest.mark.parametrize("B,Hkv,n_qtiles,g", [
    (4, 8, 16, 4), (8, 16, 8, 1), (8, 1, 8, 16), (1, 2, 1, 2), (3, 5, 7, 3), (2, 7, 3, 1),
    (7, 5, 2, 1), (5, 7, 3, 1), (1, 1, 1, 1), (13, 3, 5, 1), (9, 9, 2, 2), (2, 2, 40, 1)])
def test_work_numbering_is_a_bijection(B, Hkv, n_qtiles, g):
    total = B * Hkv * n_qtiles * g
    seen = set()
    for w in range(total):
        pair, qtile, hg = work_item(w, B, Hkv, n_qtiles, g)
        assert 0 <= pair < B * Hkv and 0 <= qtile < n_qtiles and 0 <= hg < g
        seen.add((pair, qtile, hg))
    assert len(seen) == total


def wave_slots(P, Nq, W, n_sink, q_tile0, qb, BN=64, BM=256):
    """Tiles visited by the wave owning query block qb of the work-group at
    q_tile0 (causal), or None when the wave has no rows."""
    Nk = P + Nq
    q_last = min(q_tile0 + BM, Nq) - 1
    n_tiles = min(-(-Nk // BN), (P + q_last) // BN + 1)
    sink_tiles = min(-(-n_sink // BN), n_tiles) if (W > 0 and n_sink > 0) else 0
    win_lo = max(max(P + q_tile0 - W + 1, 0) // BN, sink_tiles) if W > 0 else 0
    n_slots = sink_tiles + max(n_tiles - win_lo, 0)

    def tile_of(j):
        return j if j < sink_tiles else win_lo + (j - sink_tiles)

    def slot_of(t):
        return t if t < sink_tiles else t - win_lo + sink_tiles

    qw0 = q_tile0 + qb * 32
    if qw0 >= Nq:
        return None
    last = min(n_tiles, (P + qw0 + 31) // BN + 1) - 1
    w_end, w_first, gap = slot_of(last) + 1, 0, False
    if W > 0:
        t_w = max(P + qw0 - W + 1, 0) // BN
        if sink_tiles == 0:
            w_first = slot_of(t_w)
        else:
            ws = slot_of(t_w) if t_w >= sink_tiles else 0
            if sink_tiles < ws < w_end:
                gap, w_first = True, ws
    slots = set(range(w_first, w_end)) | (set(range(sink_tiles)) if gap else set())
    assert all(0 <= j < n_slots for j in slots)
    if gap:
        assert w_first > sink_tiles  # the loop needs one idle step before the window
    return {tile_of(j) for j in slots}


@pytest.mark.parametrize("P,Nq,W,n_sink", [
    (0, 700, 200, 4), (0, 1200, 300, 70), (0, 600, 64, 1), (100, 500, 130, 3),
    (0, 1100, 1024, 4), (0, 520, 100, 130), (300, 400, 500, 0), (0, 900, 257, 64)])
def test_window_slots_cover_every_visible_tile(P, Nq, W, n_sink):
    BN, BM = 64, 256
    for q_tile0 in range(0, Nq, BM):
        for qb in range(BM // 32):
            tiles = wave_slots(P, Nq, W, n_sink, q_tile0, qb, BN, BM)
            if tiles is None:
                continue
            qw0 = q_tile0 + qb * 32
            need = set()
            for i in range(qw0, min(qw0 + 32, Nq)):
                pq = P + i
                lo = max(pq - W + 1, 0)
                need.update(range(lo // BN, pq // BN + 1))
                need.update(range(0, (min(n_sink, pq + 1) + BN - 1) // BN))
            assert need <= tiles, (q_tile0, qb, sorted(need - tiles))
