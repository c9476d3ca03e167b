"""Pins of the oracle's paged-cache view (design reading: a pool of P-row
pages and a per-sequence block table, the layout behind the PagedAttention
the deployment guides name). The checks rest on the layout's definition,
done here with plain loops: scattering a contiguous cache into shuffled pages
and gathering it back returns every sequence's rows; attention over the
gathered rows is the contiguous result bit for bit."""
import numpy as np

import oracle


def _scatter(seqs, P, n_pages, rng):
    """Place each sequence's rows into shuffled pages with a loop over tokens."""
    max_pages = max((len(r) + P - 1) // P for r in seqs)
    pool = np.full((n_pages * P, seqs[0].shape[1]), np.nan)
    free = list(rng.permutation(n_pages))
    table = np.full((len(seqs), max_pages), -1, dtype=np.int32)
    for b, r in enumerate(seqs):
        for j in range((len(r) + P - 1) // P):
            table[b, j] = free.pop()
        for t in range(len(r)):
            pool[table[b, t // P] * P + t % P] = r[t]
    return pool, table


def test_gather_returns_every_sequence_in_token_order():
    rng = np.random.default_rng(0)
    for P in (32, 64, 96):
        seqs = [rng.standard_normal((n, 576)) for n in (1, P - 1, P, P + 1, 5 * P + 7)]
        pool, table = _scatter(seqs, P, 40, rng)
        for b, r in enumerate(seqs):
            assert np.array_equal(oracle.paged_rows(pool, table, P, b, len(r)), r)


def test_single_page_table_is_the_contiguous_layout():
    rng = np.random.default_rng(1)
    rows = rng.standard_normal((200, 576))
    # one page per sequence, pages in order: row t of sequence b at b*P + t
    P = 100
    table = np.array([[0], [1]], dtype=np.int32)
    assert np.array_equal(oracle.paged_rows(rows, table, P, 1, 60), rows[100:160])


def test_decode_over_pages_equals_contiguous_decode():
    rng = np.random.default_rng(2)
    H = 2
    seqs = [rng.standard_normal((n, 576)) for n in (3, 70, 129)]
    q_nope = rng.standard_normal((3, H, 128))
    q_pe = rng.standard_normal((3, H, 64))
    w_uk = rng.standard_normal((H, 128, 512)) / np.sqrt(512)
    w_uv = rng.standard_normal((H, 512, 128)) / np.sqrt(512)
    pool, table = _scatter(seqs, 32, 16, rng)
    o1, l1 = oracle.decode_problem(lambda b: seqs[b], q_nope, q_pe, w_uk, w_uv, 3, H)
    o2, l2 = oracle.decode_problem(lambda b: oracle.paged_rows(pool, table, 32, b, len(seqs[b])),
                                   q_nope, q_pe, w_uk, w_uv, 3, H)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
