"""Pins of the oracle's whole-block helpers, oracle.copy_blocks and oracle.swap_blocks, against
hand-worked expected bytes and against what the pages fix for them ("vllm-project-vllm -- L2",
section 9 "Memory Management": blocks are shared copy-on-write and a writer first moves to a
private copy; a preempted sequence's blocks are swapped to CPU memory and back; section 11 step 5:
a fork is a table update, the data copy happens only on the write).  CPU only.

Each case is built so that a plausible slip in either helper fails it: source and destination
exchanged, the swap direction inverted, device and host ids exchanged, or a copy that reads a
block another copy of the same call has already overwritten.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.block_manager import OK, BlockManagerModel

BS, HKV, D = 4, 2, 8


def filled_pools(num_blocks, dtype=torch.bfloat16):
    """K block b holds the value 10 + b in every element, V block b holds 100 + b (exact in bf16
    and in uint8 codes), so every block's origin can be read off any of its bytes."""
    k = torch.empty((num_blocks, BS, HKV, D), dtype=dtype)
    v = torch.empty_like(k)
    for b in range(num_blocks):
        k[b] = 10 + b
        v[b] = 100 + b
    return k, v


def block_ids(pool):
    """The constant each block holds (asserting that it is constant)."""
    flat = pool.view(pool.shape[0], -1).to(torch.float64)
    assert torch.all(flat == flat[:, :1]), "a block holds mixed contents"
    return [int(x) for x in flat[:, 0].tolist()]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.uint8])
def test_copy_blocks_hand_worked(dtype):
    """Pairs (0 -> 3), (2 -> 1) on five blocks: block 3 becomes old block 0 and block 1 old
    block 2; blocks 0, 2 and 4 are untouched.  Exchanging source and destination would give
    K = [13, 11, 11, 13, 14] instead."""
    k, v = filled_pools(5, dtype)
    oracle.copy_blocks(k, v, np.array([0, 2]), np.array([3, 1]))
    assert block_ids(k) == [10, 12, 12, 10, 14]
    assert block_ids(v) == [100, 102, 102, 100, 104]


def test_copy_blocks_reads_the_pools_as_they_were():
    """(0 -> 1) and (1 -> 2) in one call: block 2 receives the OLD block 1, not the block 0 that
    the first pair has just written there (the copies of one call all read the pre-call pools).
    A copy loop that read the live pool would give [10, 10, 10, 13]."""
    k, v = filled_pools(4)
    oracle.copy_blocks(k, v, [0, 1], [1, 2])
    assert block_ids(k) == [10, 10, 11, 13]
    assert block_ids(v) == [100, 100, 101, 103]


def gather(pool, table, n):
    """Logical tokens 0..n-1 of a sequence through its block table: [n, Hkv, D]."""
    return torch.stack([pool[table[t // BS], t % BS] for t in range(n)])


def test_copy_on_write_through_the_block_manager_model():
    """The worked trace, block_size 4 and lowest free block first:
        add(A, 6)     A = [0, 1]      (tokens 0..5)
        fork(A -> B)  B = [0, 1]      no data moves (a table update)
        append(B)     position 6 falls in shared block 1: B moves to block 2, copy (1 -> 2)
    After copy_blocks(1 -> 2), B's six logical tokens read through B's table are byte-equal to
    A's, A's blocks are unchanged, and the new token can then be written into block 2 alone."""
    m = BlockManagerModel(6, BS)
    assert m.add("A", 6) == OK and m.seqs["A"]["blocks"] == [0, 1]
    assert m.fork("A", "B") == OK
    st, slot, src, dst = m.append("B")
    assert (st, slot, src, dst) == (OK, 2 * BS + 2, 1, 2)

    g = torch.Generator().manual_seed(7)
    k = torch.randn((6, BS, HKV, D), generator=g).to(torch.bfloat16)
    v = torch.randn((6, BS, HKV, D), generator=g).to(torch.bfloat16)
    k[2] = float("nan")                  # block 2 was free: stale contents
    v[2] = float("nan")
    k_before, v_before = k.clone(), v.clone()
    oracle.copy_blocks(k, v, [src], [dst])

    ta, tb = m.seqs["A"]["blocks"], m.seqs["B"]["blocks"]
    assert tb == [0, 2]
    for pool, before in ((k, k_before), (v, v_before)):
        assert torch.equal(gather(pool, tb, 6).view(torch.int16), gather(before, ta, 6).view(torch.int16))
        for b in (0, 1, 3, 4, 5):        # only the destination changed
            assert torch.equal(pool[b].view(torch.int16), before[b].view(torch.int16))

    # the new token at B's slot lands in B's private block only; A's token 6 slot is untouched
    kn = torch.full((1, HKV, D), 7.0).to(torch.bfloat16)
    oracle.kv_write(kn, kn, k, v, np.array([slot], dtype=np.int64))
    assert torch.equal(k[2, 2], kn[0]) and torch.equal(k[1, 2], k_before[1, 2])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.uint8])
def test_swap_out_and_in_hand_worked(dtype):
    """Device pool of 8 blocks, host pool of 4, block_size 4, lowest free first:
        add(X, 4) X = [0];  add(S, 9) S = [1, 2, 3];  release(X) frees block 0
        swap_out(S)   pairs (1 -> host 0), (2 -> host 1), (3 -> host 2); device 1..3 freed
        add(Y, 13)    Y takes device [0, 1, 2, 3]   (S's old blocks are overwritten)
        swap_in(S)    pairs (host 0 -> 4), (host 1 -> 5), (host 2 -> 6)
    Expected bytes at each step are the block constants of filled_pools."""
    m = BlockManagerModel(8, BS, num_host_blocks=4)
    assert m.add("X", 4) == OK and m.add("S", 9) == OK and m.seqs["S"]["blocks"] == [1, 2, 3]
    assert m.release("X") == OK
    k, v = filled_pools(8, dtype)
    hk = torch.zeros((4, BS, HKV, D), dtype=dtype)
    hv = torch.zeros_like(hk)
    hk[3] = 55                            # an unused host block keeps its bytes
    hv[3] = 55

    st, pairs = m.swap_out("S")
    assert st == OK and pairs == [(1, 0), (2, 1), (3, 2)]
    oracle.swap_blocks(k, v, hk, hv, [d for d, _ in pairs], [h for _, h in pairs], to_host=True)
    assert block_ids(hk) == [11, 12, 13, 55] and block_ids(hv) == [101, 102, 103, 55]
    assert block_ids(k) == [10 + b for b in range(8)]          # swap-out leaves the device pool as is

    assert m.add("Y", 13) == OK and m.seqs["Y"]["blocks"] == [0, 1, 2, 3]
    for b in range(4):                                         # Y's prompt overwrites them
        k[b] = 40 + b
        v[b] = 140 + b

    st, pairs = m.swap_in("S")
    assert st == OK and pairs == [(0, 4), (1, 5), (2, 6)]
    oracle.swap_blocks(k, v, hk, hv, [d for _, d in pairs], [h for h, _ in pairs], to_host=False)
    assert block_ids(k) == [40, 41, 42, 43, 11, 12, 13, 17]
    assert block_ids(v) == [140, 141, 142, 143, 101, 102, 103, 107]
    assert block_ids(hk) == [11, 12, 13, 55]                   # swap-in leaves the host pool as is
    # S's nine logical tokens, read through its new table, are its original ones
    ok, rows, lens = m.table(["S"], 3)
    assert ok == OK and rows == [[4, 5, 6]] and lens == [9]
    ref_k, _ = filled_pools(8, dtype)
    assert torch.equal(gather(k, rows[0], 9), gather(ref_k, [1, 2, 3], 9))


def test_swap_round_trip_restores_random_contents():
    """Random bytes survive a swap-out to permuted host ids and a swap-in to other device ids;
    every byte outside the targets is unchanged in both directions."""
    rng = np.random.default_rng(3)
    g = torch.Generator().manual_seed(3)
    k = torch.randint(0, 256, (12, BS, HKV, D), generator=g, dtype=torch.uint8)
    v = torch.randint(0, 256, (12, BS, HKV, D), generator=g, dtype=torch.uint8)
    hk = torch.randint(0, 256, (9, BS, HKV, D), generator=g, dtype=torch.uint8)
    hv = torch.randint(0, 256, (9, BS, HKV, D), generator=g, dtype=torch.uint8)
    dev = rng.permutation(12)[:5]
    host = rng.permutation(9)[:5]
    k0, v0, hk0, hv0 = k.clone(), v.clone(), hk.clone(), hv.clone()
    oracle.swap_blocks(k, v, hk, hv, dev, host, to_host=True)
    for i in range(9):
        want_k = k0[dev[list(host).index(i)]] if i in host else hk0[i]
        want_v = v0[dev[list(host).index(i)]] if i in host else hv0[i]
        assert torch.equal(hk[i], want_k) and torch.equal(hv[i], want_v)
    assert torch.equal(k, k0) and torch.equal(v, v0)
    back = np.setdiff1d(np.arange(12), dev)[:5]               # other device blocks
    oracle.swap_blocks(k, v, hk, hv, back, host, to_host=False)
    for j, d in enumerate(back):
        assert torch.equal(k[d], k0[dev[j]]) and torch.equal(v[d], v0[dev[j]])
    untouched = np.setdiff1d(np.arange(12), back)
    assert torch.equal(k[untouched], k0[untouched]) and torch.equal(v[untouched], v0[untouched])
