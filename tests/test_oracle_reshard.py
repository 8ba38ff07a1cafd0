"""Pins of the oracle's reshard-to-a-smaller-group plan (reshard_after_forward
as an integer k: "FSDP2's parameter lifecycle...", section "Reshard policy:
pay for the memory, or pay for the communication again").

The two ends are fixed by the page itself: k = N is full resharding (a rank
keeps only its own 1/N shard, the slice the FLAT gather writes) and k = 1 is
no resharding (a rank keeps the whole gathered buffer). In between, every
group of k consecutive ranks must hold the whole buffer exactly once, every
N-way shard must land in exactly one slice index, and the slices a rank
assembles from its sources must equal the same range of the buffer the N
ranks' FLAT gathers build. Each pin is checked against a construction other
than the reshard code (the flat gather, brute-force coverage)."""
import random

import numpy as np
import pytest

import oracle
from oracle.plan import plan_flat, reshard_slice


def _divisors(n):
    return [k for k in range(1, n + 1) if n % k == 0]


@pytest.mark.parametrize("N", [1, 2, 4, 8, 64])
def test_group_of_world_size_is_the_own_shard(ora, N):
    numels = [1000, 77, 4096]
    for r in range(N):
        p = plan_flat(numels, N, r, 8)
        s = reshard_slice(p, N)
        assert (s.slice_index, s.slice_off, s.slice_len) == (r, r * p.S, p.S)
        assert (s.first_source, s.n_sources, s.owner_slice, s.own_off) == (r, 1, r, 0)
        assert s.retained_bytes == 2 * p.S  # the bf16 parameter share of the 16 B/param ledger
        # writing the own shard into the kept slice == the flat gather's own slice
        par = np.arange(p.S, dtype=np.uint16) ^ 0x3C00
        sl = np.full(s.slice_len, 0xABCD, np.uint16)
        ora.gather_to_slice(par, s.own_off, sl)
        full = np.full(p.T, 0xABCD, np.uint16)
        ora.gather(par, r, full)
        assert np.array_equal(sl, full[s.slice_off:s.slice_off + s.slice_len])


@pytest.mark.parametrize("N", [1, 3, 8, 64])
def test_group_of_one_is_the_whole_buffer(ora, N):
    numels = [123_457, 9]
    for r in range(N):
        p = plan_flat(numels, N, r, 8)
        s = reshard_slice(p, 1)
        assert (s.slice_index, s.slice_off, s.slice_len) == (0, 0, p.T)
        assert (s.first_source, s.n_sources, s.owner_slice, s.own_off) == (0, N, 0, r * p.S)
        assert s.retained_bytes == 2 * p.T
        par = (np.arange(p.S, dtype=np.uint32) * 2654435761 >> 16).astype(np.uint16)
        sl = np.full(p.T, 0x5A5A, np.uint16)
        ora.gather_to_slice(par, s.own_off, sl)
        full = np.full(p.T, 0x5A5A, np.uint16)
        ora.gather(par, r, full)  # the flat gather, an independent function
        assert np.array_equal(sl, full)


def test_groups_tile_the_buffer_and_shards_land_once():
    rng = random.Random(5)
    for _ in range(40):
        N = rng.choice([1, 2, 4, 6, 8, 12, 16, 24, 64])
        numels = [rng.randrange(0, 5000) for _ in range(rng.randrange(1, 6))]
        align = rng.choice([1, 8, 128])
        for k in _divisors(N):
            plans = [plan_flat(numels, N, r, align) for r in range(N)]
            T, S = plans[0].T, plans[0].S
            sl = [reshard_slice(p, k) for p in plans]
            for g in range(N // k):  # each group of k consecutive ranks holds [0, T) exactly once
                cover = np.zeros(T, np.int32)
                for r in range(g * k, (g + 1) * k):
                    cover[sl[r].slice_off:sl[r].slice_off + sl[r].slice_len] += 1
                assert np.all(cover == 1), (N, k, g)
            holders = {}
            for r, s in enumerate(sl):
                # the own shard sits inside its owner slice at own_off
                assert s.owner_slice * s.slice_len + s.own_off == r * S
                assert 0 <= s.own_off and s.own_off + S <= s.slice_len
                # the kept slice is exactly its sources' shards, in order
                assert s.slice_off == s.first_source * S and s.slice_len == s.n_sources * S
                for q in range(s.first_source, s.first_source + s.n_sources):
                    holders.setdefault(q, set()).add(r)
            for q in range(N):  # shard q is kept by one rank in every group, the one holding slice owner(q)
                assert len(holders[q]) == N // k
                assert all(sl[r].slice_index == sl[q].owner_slice for r in holders[q])


def test_assembled_slices_equal_the_flat_gathered_buffer(ora):
    N, numels = 8, [100_003, 4093, 1]
    rng = np.random.default_rng(3)
    plans = [plan_flat(numels, N, r, 8) for r in range(N)]
    T, S = plans[0].T, plans[0].S
    params = [rng.integers(0, 1 << 16, S, dtype=np.uint16) for _ in range(N)]
    full = np.zeros(T, np.uint16)
    for r in range(N):
        ora.gather(params[r], r, full)
    for k in _divisors(N):
        for r in range(N):
            s = reshard_slice(plans[r], k)
            kept = np.full(s.slice_len, 0xFFFF, np.uint16)
            ora.gather_slice([params[q] for q in range(s.first_source, s.first_source + s.n_sources)], kept)
            assert np.array_equal(kept, full[s.slice_off:s.slice_off + s.slice_len]), (k, r)
            # and the slice that holds r's own shard, written by r, equals the same range
            own = np.zeros(s.slice_len, np.uint16)
            ora.gather_to_slice(params[r], s.own_off, own)
            lo = s.owner_slice * s.slice_len
            assert np.array_equal(own[s.own_off:s.own_off + S], full[lo + s.own_off:lo + s.own_off + S])


def test_retained_bytes_fall_from_no_reshard_to_full_reshard():
    """The page's trade: keeping more after forward (smaller reshard degree of
    freedom) costs memory and saves backward AllGather traffic. Retained bf16
    bytes are 2*T/k: k = 1 keeps the whole model (2*T), k = N keeps 2*S; at the
    Llama-70B shape over 64 ranks in nodes of 8, resharding within the node
    keeps 1/8 of the model per rank."""
    from synth.shapes import llama_70b
    numels = llama_70b()
    p = plan_flat(numels, 64, 5, 128)
    got = [reshard_slice(p, k).retained_bytes for k in (1, 2, 4, 8, 16, 32, 64)]
    assert got == sorted(got, reverse=True)
    assert got[0] == 2 * p.T and got[-1] == 2 * p.S
    assert got[3] == 2 * p.T // 8 == 17_638_426_624
    node = reshard_slice(p, 8)
    assert node.slice_index == 5 and node.first_source == 40 and node.n_sources == 8  # ranks 40..47's shards
    assert node.owner_slice == 0 and node.own_off == 5 * p.S  # rank 5's own shard lies in slice 0


@pytest.mark.parametrize("N,k", [(8, 3), (8, 0), (8, 9), (6, 4)])
def test_group_size_must_divide_the_world(N, k):
    with pytest.raises(ValueError):
        reshard_slice(plan_flat([100], N, 0), k)


def test_per_tensor_plans_have_no_flat_slices():
    with pytest.raises(ValueError):
        reshard_slice(oracle.plan_per_tensor([100], 4, 0), 2)
