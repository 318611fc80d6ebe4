"""Pins of the oracle's batch geometry and guard policy (hand-counted cases and
the limits the definition fixes)."""
import oracle


def test_request_offsets_hand_counted():
    # requests (L, q_len) = (5, 3), (7, 7), (4, 1) with g = 2:
    # groups ceil(3/2) = 2, ceil(7/2) = 4, 1
    assert oracle.request_offsets([5, 7, 4], [3, 7, 1], 2) == ([0, 5, 12], [0, 3, 10], [0, 2, 6])


def test_guarded_groups_hand_counted():
    # prefill L = q_len = 100, g = 4: group m ends at 4m + 3, prefix 4(m+1) keys
    assert oracle.guarded_groups(100, 100, 4, 10) == 2   # prefixes 4, 8 <= 10 < 12
    assert oracle.guarded_groups(100, 100, 4, 12) == 3
    # decode-like: 10 rows at the end of 100 keys (positions 90..99), g = 4:
    # prefixes 94, 98, 100
    assert oracle.guarded_groups(100, 10, 4, 93) == 0
    assert oracle.guarded_groups(100, 10, 4, 95) == 1
    assert oracle.guarded_groups(100, 10, 4, 99) == 2
    assert oracle.guarded_groups(100, 10, 4, 100) == 3   # the short last group too


def test_guarded_groups_limits():
    for L, q, g in [(1, 1, 1), (50, 50, 3), (1000, 7, 16), (4096, 4096, 4)]:
        G = -(-q // g)
        assert oracle.guarded_groups(L, q, g, 0) == 0
        assert oracle.guarded_groups(L, q, g, L) == G
        prev = 0
        for guard in range(0, L + 2, max(1, L // 37)):
            n = oracle.guarded_groups(L, q, g, guard)
            assert prev <= n <= G
            prev = n
