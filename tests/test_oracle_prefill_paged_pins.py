"""Pins of the paged prefill oracle (oracle.prefill_mha_paged).  CPU only.

Paging is address translation: position i of sequence b is row i mod P of
page block_table[b, i // P] ([intelliparadigm.com .../2131745] section
5.1).  The pins tie the paged oracle to the contiguous prefill oracle
(pinned on its own in tests/test_oracle_prefill_pins.py) and to that
mapping, written out as a brute-force loop:
  * an identity table over a pool laid out like the contiguous cache gives
    the contiguous oracle's outputs and bytes;
  * a random table gives the same outputs, and every appended row sits at
    the page and row the table names, every other pool row untouched;
  * an invalid entry among a sequence's pages gives NaN rows for that
    sequence only, and appends exactly the rows of its valid pages."""
import numpy as np
import pytest

import oracle
from tests.test_oracle_prefill_pins import prompt


def pools(n_pages, Hkv, P, D, dtype, fill):
    kp = np.full((n_pages, Hkv, P, D), fill, dtype=dtype)
    return kp, kp.copy()


def poison_of(dt):
    return np.uint16(0x7fc0) if dt == "bf16" else np.float16(np.nan)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_identity_table_is_the_contiguous_prefill(dt):
    B, H, Hkv, D, S, P = 2, 4, 2, 8, 11, 4
    npp = (S + P - 1) // P                  # pages per sequence
    case, q, kn, vn, bias, kc, vc = prompt(dt, B, H, Hkv, D, S, npp * P, seed=21)
    lens = np.array([S, 6], np.int32)
    ref = oracle.prefill_mha(q, kn, vn, bias, kc, vc, lens, H, Hkv, D, dt)
    kp, vp = pools(B * npp, Hkv, P, D, q.dtype, poison_of(dt))
    table = np.arange(B * npp, dtype=np.int32).reshape(B, npp)
    out = oracle.prefill_mha_paged(q, kn, vn, bias, kp, vp, table, lens, H, Hkv, D, dt)
    assert np.array_equal(out, ref, equal_nan=True)
    # page i of sequence b holds its positions [i P, (i + 1) P)
    for which, pool, cache in ((0, kp, kc), (1, vp, vc)):
        as_cache = pool.reshape(B, npp, Hkv, P, D).swapaxes(1, 2).reshape(B, Hkv, npp * P, D)
        assert as_cache.tobytes() == cache.tobytes(), which


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_random_table_places_every_row(dt):
    B, H, Hkv, D, S, P = 3, 6, 3, 8, 13, 4
    case, q, kn, vn, bias, kc, vc = prompt(dt, B, H, Hkv, D, S, S, seed=23)
    lens = np.array([13, 1, 9], np.int32)
    ref = oracle.prefill_mha(q, kn, vn, bias, kc, vc, lens, H, Hkv, D, dt)
    max_pages = (S + P - 1) // P
    n_pages = B * max_pages + 3
    perm = np.random.default_rng(4).permutation(n_pages)
    table = np.full((B, max_pages), -1, np.int32)
    used = 0
    for b in range(B):
        for i in range((int(lens[b]) + P - 1) // P):
            table[b, i] = perm[used]
            used += 1
    kp, vp = pools(n_pages, Hkv, P, D, q.dtype, poison_of(dt))
    kp0, vp0 = kp.copy(), vp.copy()
    out = oracle.prefill_mha_paged(q, kn, vn, bias, kp, vp, table, lens, H, Hkv, D, dt)
    for b in range(B):
        Sb = int(lens[b])
        assert np.array_equal(out[b, :Sb], ref[b, :Sb])
    written = np.zeros(kp.shape[:3], dtype=bool)    # [page, head, row]
    for b in range(B):
        for t in range(int(lens[b])):
            pg, r = table[b, t // P], t % P
            written[pg, :, r] = True
            assert kp[pg, :, r].tobytes() == kc[b, :, t].tobytes()
            assert vp[pg, :, r].tobytes() == vc[b, :, t].tobytes()
    assert kp[~written].tobytes() == kp0[~written].tobytes()
    assert vp[~written].tobytes() == vp0[~written].tobytes()


def test_invalid_page_gives_nan_rows_and_appends_the_valid_pages():
    dt = "f16"
    B, H, Hkv, D, S, P = 2, 2, 1, 8, 12, 4
    case, q, kn, vn, bias, kc, vc = prompt(dt, B, H, Hkv, D, S, S, seed=25)
    ref = oracle.prefill_mha(q, kn, vn, bias, kc, vc, None, H, Hkv, D, dt)
    n_pages = 8
    table = np.array([[0, 1, 2], [3, 99, 5]], np.int32)     # sequence 1, page 1 (positions 4..7) invalid
    kp, vp = pools(n_pages, Hkv, P, D, q.dtype, np.float16(0))
    out = oracle.prefill_mha_paged(q, kn, vn, bias, kp, vp, table, None, H, Hkv, D, dt)
    assert np.array_equal(out[0], ref[0])
    assert np.isnan(out[1]).all()
    for t in range(S):
        if t // P == 1:
            continue
        pg = table[1, t // P]
        assert kp[pg, :, t % P].tobytes() == kc[1, :, t].tobytes()
    assert not kp[4].any() and not kp[6].any() and not kp[7].any()   # pages no valid entry names
