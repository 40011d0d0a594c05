"""Pins of the paged-cache oracle (oracle.paged) against facts fixed outside it:

  * a hand-placed example whose key rows are listed literally, not derived;
  * the identity layout (each sequence's blocks consecutive, in order) is the
    contiguous cache, so the result must equal the plain definition (itself pinned by
    brute force and a library routine);
  * renumbering the physical blocks, or changing pool rows no sequence owns, changes
    nothing;
  * a sequence without keys gives O = 0 and lse = -inf;
  * planted mistakes in the gather (row and block index, head, table row) are caught.
"""
import numpy as np
import pytest

import oracle
import oracle.paged as op


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_hand_placed_example():
    # pool of 3 blocks of 2 keys, 1 head, d = 3; sequence 0 owns blocks [2, 0] and 3
    # keys: key 0 = pool[2, 0, 0], key 1 = pool[2, 0, 1], key 2 = pool[0, 0, 0].
    rng = np.random.default_rng(1)
    kp, vp = _rand(rng, 3, 1, 2, 3), _rand(rng, 3, 1, 2, 3)
    q = _rand(rng, 1, 1, 2, 3)
    table = np.array([[2, 0]])
    keys = np.stack([kp[2, 0, 0], kp[2, 0, 1], kp[0, 0, 0]])
    vals = np.stack([vp[2, 0, 0], vp[2, 0, 1], vp[0, 0, 0]])
    o, lse = op.paged_attention_forward(q, kp, vp, table, np.array([3]), scale=0.7)
    s = 0.7 * q[0, 0] @ keys.T
    w = np.exp(s - s.max(axis=1, keepdims=True))
    np.testing.assert_allclose(o[0, 0], (w @ vals) / w.sum(axis=1, keepdims=True), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(np.exp(s).sum(axis=1)), rtol=0, atol=1e-14)


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_identity_layout_is_the_contiguous_cache(bs):
    rng = np.random.default_rng(bs)
    B, H, Nq, d, mb = 3, 2, 5, 8, 4
    n = mb * bs
    q, k, v = _rand(rng, B, H, Nq, d), _rand(rng, B, H, n, d), _rand(rng, B, H, n, d)
    # sequence b owns blocks b*mb .. b*mb+mb-1; block c of sequence b holds keys
    # c*bs .. c*bs+bs-1 of every head
    kp = k.reshape(B, H, mb, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * mb, H, bs, d)
    vp = v.reshape(B, H, mb, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * mb, H, bs, d)
    table = np.arange(B * mb).reshape(B, mb)
    for lens in ([n, n, n], [n, 1, n - 1]):
        o, lse = op.paged_attention_forward(q, kp, vp, table, np.array(lens), scale=0.3)
        for b, L in enumerate(lens):
            o_ref, l_ref = oracle.attention_forward(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L],
                                                    causal=False, scale=0.3)
            np.testing.assert_allclose(o[b], o_ref[0], rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[b], l_ref[0], rtol=0, atol=1e-13)


def _scattered(seed, B=3, H=2, Nq=3, d=8, bs=4, lens=(9, 4, 1), spare=3):
    rng = np.random.default_rng(seed)
    per = [-(-L // bs) for L in lens]
    nb = sum(per) + spare
    perm = rng.permutation(nb)
    mb = max(per)
    table = np.full((B, mb), -1)
    at = 0
    for b, c in enumerate(per):
        table[b, :c] = perm[at:at + c]
        at += c
    return (_rand(rng, B, H, Nq, d), _rand(rng, nb, H, bs, d), _rand(rng, nb, H, bs, d), table,
            np.array(lens))


def test_block_renumbering_invariance():
    q, kp, vp, table, lens = _scattered(3)
    o, lse = op.paged_attention_forward(q, kp, vp, table, lens, scale=0.5)
    perm = np.random.default_rng(9).permutation(kp.shape[0])      # new id of block i is perm[i]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    o2, lse2 = op.paged_attention_forward(q, kp2, vp2, table2, lens, scale=0.5)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_unowned_rows_do_not_matter():
    q, kp, vp, table, lens = _scattered(4)
    bs = kp.shape[2]
    o, lse = op.paged_attention_forward(q, kp, vp, table, lens, scale=0.5)
    owned = np.zeros(kp.shape[:3], dtype=bool)
    for b, L in enumerate(lens):
        for j in range(L):
            owned[table[b, j // bs], :, j % bs] = True
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[~owned] = 1e3
    vp2[~owned] = -1e6
    o2, lse2 = op.paged_attention_forward(q, kp2, vp2, table, lens, scale=0.5)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_empty_sequence():
    q, kp, vp, table, _ = _scattered(5)
    o, lse = op.paged_attention_forward(q, kp, vp, table, np.array([9, 0, 1]), scale=0.5)
    assert np.all(o[1] == 0) and np.all(lse[1] == -np.inf)
    assert np.all(np.isfinite(o[0])) and np.all(np.isfinite(lse[2]))


def test_rejects_lengths_and_entries_outside():
    q, kp, vp, table, _ = _scattered(6)
    with pytest.raises(ValueError):
        op.paged_attention_forward(q, kp, vp, table, np.array([13, 1, 1]), scale=0.5)
    bad = table.copy()
    bad[0, 0] = kp.shape[0]
    with pytest.raises(ValueError):
        op.paged_attention_forward(q, kp, vp, bad, np.array([9, 4, 1]), scale=0.5)


def _pins_pass():
    try:
        test_hand_placed_example()
        for bs in (1, 4, 16):
            test_identity_layout_is_the_contiguous_cache(bs)
        test_block_renumbering_invariance()
        test_unowned_rows_do_not_matter()
    except AssertionError:
        return False
    return True


def _gather_mutant(kind):
    def gather(pool, block_table, b, h, n_keys, block_size):
        j = np.arange(n_keys)
        row = j // block_size if kind == "row_div" else j % block_size
        blk_idx = j % block_size if kind == "block_mod" else j // block_size
        if kind == "block_off_by_one":
            blk_idx = np.minimum(blk_idx + 1, block_table.shape[1] - 1)
        tb = b if kind != "table_row0" else 0
        blocks = np.asarray(block_table)[tb, blk_idx]
        if kind == "physical_is_logical":
            blocks = blk_idx + b * block_table.shape[1]
            blocks = np.minimum(blocks, pool.shape[0] - 1)
        hh = 0 if kind == "head0" else h
        if kind == "reversed_rows":
            row = block_size - 1 - row
        return pool[blocks, hh, row]
    return gather


@pytest.mark.parametrize("kind", ["row_div", "block_mod", "block_off_by_one", "table_row0",
                                  "physical_is_logical", "head0", "reversed_rows"])
def test_pins_reject_gather_mutant(kind, monkeypatch):
    monkeypatch.setattr(op, "gather_keys", _gather_mutant(kind))
    assert not _pins_pass(), kind


def test_unmutated_gather_passes():
    assert _pins_pass()
