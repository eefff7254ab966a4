"""Pins for the oracle's reading of paged caches (CPU only).

A paged cache (tokamax "Supported Ops and Hardware", Attention Variants:
lightning_indexer over a paged KV cache) stores slot s of sequence r at pool
row block_table[r, s // page_size] * page_size + s % page_size.  The oracle's
unpage is checked against the seeded generator's own page scatter (an
independent loop in the other direction), a hand-checked row, and the
identity table, for which unpaging is a plain reshape.
"""
import numpy as np
import torch

import oracle
import synthetic


def test_unpage_inverts_page_scatter():
    # the generator scatters a contiguous cache into pages (its own loop); unpaging must give it back,
    # for a ragged last page and for bf16, fp8-code and fp32-scale pools
    P, n_seq, n_slots = 64, 3, 150
    max_pages = -(-n_slots // P)
    n_pages = n_seq * max_pages + 4
    table = synthetic.page_table(5, 9, n_seq, max_pages, n_pages)
    assert len(set(table.flatten().tolist())) == n_seq * max_pages  # distinct pages
    g = np.random.default_rng(3)
    x = torch.from_numpy(g.standard_normal((n_seq, n_slots, 128)).astype(np.float32)).to(torch.bfloat16)
    fill = torch.full((n_pages * P, 128), 99.0, dtype=torch.bfloat16)
    pool = synthetic.scatter_pages(x, table, P, n_pages, fill)
    back = oracle.unpage(pool, table, P, n_slots)
    assert np.array_equal(back, x.view(torch.int16).numpy().view(np.uint16))
    sc = torch.from_numpy(g.standard_normal((n_seq, n_slots)).astype(np.float32))
    spool = synthetic.scatter_pages(sc, table, P, n_pages, torch.zeros(n_pages * P))
    assert np.array_equal(oracle.unpage(spool, table, P, n_slots), sc.numpy())
    # a hand-checked slot: sequence 2, slot 130 -> page table[2, 2], row 2 of it
    row = int(table[2, 2]) * P + 2
    assert np.array_equal(pool[row].view(torch.int16).numpy(), x[2, 130].view(torch.int16).numpy())


def test_unpage_identity_table_is_a_reshape():
    P, n_seq, max_pages = 64, 2, 3
    table = torch.arange(n_seq * max_pages, dtype=torch.int32).view(n_seq, max_pages)
    pool = np.arange(n_seq * max_pages * P * 4, dtype=np.float32).reshape(-1, 4)
    back = oracle.unpage(pool, table, P, max_pages * P)
    assert np.array_equal(back, pool.reshape(n_seq, max_pages * P, 4))
