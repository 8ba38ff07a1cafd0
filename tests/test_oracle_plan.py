"""Pins of the oracle's shard plan and persistent-byte ledger.

Checked against numbers the pages print (tests/golden/ledger_numbers.json),
closed-form sizes of the model shapes, and a brute-force coverage check over
random tensor lists.
"""
import json
import os
import random

import pytest

from oracle.plan import plan_flat, plan_per_tensor, roundup
from synth import shapes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ledger_numbers.json")))


def test_bytes_per_param_is_16():
    g = GOLD["bytes_per_param"]
    assert sum(g["parts"]) == g["value"] == 16
    p = plan_flat([1024], 1, 0)
    assert p.persistent_bytes == 16 * 1024


def test_tiny_plan_closed_form():
    p = plan_flat(shapes.tiny(), 4, 1)
    assert p.T == 1_000_032 and p.S == 250_008
    assert p.T - 1_000_003 == 29
    (pc,) = p.pieces
    assert (pc.own_lo, pc.own_hi, pc.shard_off) == (250_008, 500_016, 0)
    p3 = plan_flat(shapes.tiny(), 4, 3)
    (pc3,) = p3.pieces
    # rank 3 owns [750,024, 1,000,032): 249,979 real elements, then the 29 pads
    assert (pc3.own_lo, pc3.own_hi) == (750_024, 1_000_003)
    mask = p3.padding_mask_full()
    assert sum(mask) == 29 and all(mask[1_000_003:]) and not any(mask[:1_000_003])


def test_qwen_param_count_matches_oom_message():
    sizes = shapes.qwen25_3b()
    assert len(sizes) == 434
    P = sum(sizes)
    assert P == 3_085_938_688
    # the ZeRO-0 OOM tried to allocate one fp32 model-sized buffer: 11.50 GiB
    assert round(4 * P / 2**30, 2) == GOLD["qwen3b_oom_alloc_GiB"]["value"]


def test_qwen_staircase_n4():
    sizes = shapes.qwen25_3b()
    p = plan_flat(sizes, 4, 0, 128)
    assert p.T == sum(sizes)  # every size is a multiple of 128: no padding
    assert p.S == 771_484_672
    g = GOLD["qwen3b_staircase_theory_GB_N4"]
    T, S = p.T, p.S
    zero1 = (2 + 2) * T + 12 * S  # params, grads replicated; optimizer sharded
    zero2 = 2 * T + 14 * S  # params replicated
    zero3 = p.persistent_bytes  # everything sharded: the ledger
    for key, val in (("zero1", zero1), ("zero2", zero2), ("zero3", zero3)):
        assert abs(val / 1e9 - g[key]) <= g["tolerance_GB"], (key, val / 1e9)
    assert zero3 == 16 * S


def test_llama7b_ledger_dp8():
    sizes = shapes.llama_7b()
    assert len(sizes) == 291 and sum(sizes) == 6_738_415_616
    assert sum(1 for s in sizes if s == 4096) == 65
    p = plan_flat(sizes, 8, 0, 128)
    assert p.T == 6_738_415_616 and p.S == 842_301_952
    g = GOLD["zero_GB_7b_dp8"]
    assert abs(p.persistent_bytes / 1e9 - g["zero3"]) <= 1.0  # ~14 GB per rank
    assert p.persistent_bytes == 13_476_831_232
    # the per-parameter ratios of the three stages at dp=8
    b = GOLD["zero_bytes_per_param_dp8"]
    assert (4 + 12 / 8, 2 + 14 / 8, 16 / 8) == (b["zero1"], b["zero2"], b["zero3"])
    for key in ("zero1", "zero2", "zero3"):
        assert abs(b[key] * g["params"] / 1e9 - g[key]) < 0.6
    assert GOLD["state_7b_GB"]["value"] == 16 * GOLD["state_7b_GB"]["params"] / 1e9
    assert abs(GOLD["state_70b_TB"]["value"] - 16 * GOLD["state_70b_TB"]["params"] / 1e12) < 1e-9


def test_llama7b_buckets():
    S = plan_flat(shapes.llama_7b(), 8, 0, 128).S
    B = 25_000_000
    buckets = [(o, min(B, S - o)) for o in range(0, S, B)]
    assert len(buckets) == 34 and buckets[-1][1] == 17_301_952
    assert all(o % 8 == 0 and n % 8 == 0 for o, n in buckets)


def test_llama70b_shard():
    sizes = shapes.llama_70b()
    assert len(sizes) == 723 and sum(sizes) == 70_553_706_496
    p = plan_flat(sizes, 64, 0, 128)
    assert p.S == 1_102_401_664 and p.T == sum(sizes)
    assert p.persistent_bytes == 16 * 1_102_401_664


def test_wrap_stress_pieces():
    sizes = shapes.llama_7b()
    p = plan_per_tensor(sizes, 8, 0)
    assert len(p.pieces) == 291
    lens = [pc.own_hi - pc.own_lo for pc in p.pieces]
    assert max(lens) == 16_384_000 and min(lens) == 512
    assert sum(1 for n in lens if n == 512) == 65
    assert p.S == 842_301_952  # no tensor needs padding at N*8 = 64
    assert p.persistent_bytes == 16 * p.S


def test_norm_768_over_64():
    g = GOLD["norm_768_over_64"]
    assert g["numel"] // g["world"] == g["shard_elems"] == 12
    # With a 16-byte shard granule the shard is 16 elements and 256 pad.
    p = plan_per_tensor([768], 64, 0)
    assert p.T == 1024 and p.S == 16
    reals = [plan_per_tensor([768], 64, r).pieces[0] for r in range(64)]
    assert sum(pc.real_hi - pc.real_lo for pc in reals) == 768
    assert reals[47].real_hi - reals[47].real_lo == 16 and reals[48].real_hi == reals[48].real_lo


def _tiles(spans, total):
    """True when the [start, end) spans, in order, cover [0, total) with no gap or overlap."""
    pos = 0
    for a, b in sorted(spans):
        if a != pos or b < a:
            return False
        pos = b
    return pos == total


@pytest.mark.parametrize("seed", range(20))
def test_brute_force_coverage(seed):
    rnd = random.Random(seed)
    ntens = rnd.randint(0, 12)
    numels = [rnd.choice([0, 1, 7, 8, 13, 64, 100, 768, 1000, 4097]) for _ in range(ntens)]
    world = rnd.choice([1, 2, 3, 4, 5, 8, 64])
    align = rnd.choice([1, 2, 8, 128])
    for layout in ("flat", "per_tensor"):
        cover = {}
        Ss = set()
        gathered = []  # every rank's pieces as [start, end) of the gathered buffer
        for r in range(world):
            p = plan_flat(numels, world, r, align) if layout == "flat" else plan_per_tensor(numels, world, r)
            Ss.add(p.S)
            for pc in p.pieces:
                n_pc = pc.own_hi - pc.own_lo
                gathered.append((pc.full_off, pc.full_off + n_pc))
                if layout == "flat":
                    # the gather writes the shard at r*S: a piece's two coordinates agree
                    assert pc.full_off == r * p.S + pc.shard_off
                else:
                    # inside its tensor's padded span, at the r-th of its N equal slices
                    Ti = p.padded[pc.tensor]
                    assert pc.full_off == p.offsets[pc.tensor] + r * (Ti // world)
            if layout == "per_tensor":
                # tensors packed in order; the pieces tile the shard
                assert p.offsets == [sum(p.padded[:i]) for i in range(len(numels))]
                assert _tiles([(pc.shard_off, pc.shard_off + pc.own_hi - pc.own_lo) for pc in p.pieces], p.S)
            assert p.T == world * p.S and p.S % 8 == 0
            if layout == "flat":
                assert p.T % (8 * world) == 0
                assert all(o % align == 0 for o in p.offsets)
                end = (p.offsets[-1] + numels[-1]) if numels else 0
                assert 0 <= p.T - end < 8 * world
            else:
                assert all(Ti % (8 * world) == 0 and Ti - n < 8 * world for Ti, n in zip(p.padded, numels))
            assert p.persistent_bytes == 16 * p.S
            for pc in p.pieces:
                for k in range(pc.real_lo, pc.real_hi):
                    key = (pc.tensor, k)
                    assert key not in cover
                    cover[key] = r
        assert len(Ss) == 1
        assert len(cover) == sum(numels)
        # across the ranks, pieces never overlap in the gathered buffer; with
        # per-tensor sharding they tile all of it, padding included
        gathered.sort()
        assert all(b0 <= a1 for (_a0, b0), (a1, _b1) in zip(gathered, gathered[1:]))
        if layout == "per_tensor":
            assert _tiles(gathered, p.T)


def _units(sizes, per_block, n_layers=32, per_layer=9):
    """FSDP units of the Llama-7B tensor list under a wrap policy ("FSDP2's
    parameter lifecycle...", section "Wrap granularity is the lever"): per
    block, every block is one unit and the root unit keeps the embedding,
    final norm and head; per linear, every linear sublayer is a unit of its
    own and each block's two norms stay in the block's unit."""
    emb, layers, tail = sizes[:1], sizes[1:1 + n_layers * per_layer], sizes[1 + n_layers * per_layer:]
    units = []
    for b in range(n_layers):
        blk = layers[b * per_layer:(b + 1) * per_layer]
        if per_block:
            units.append(blk)
        else:
            units += [[n] for n in blk[:7]] + [blk[7:]]
    units.append(emb + tail)
    return units


def test_wrap_units_and_ledger():
    """Per-block wrapping: 33 units (32 blocks + root), one all-gather each per
    block; per-linear wrapping: 7 units per block (the page's example counts 6
    linear sublayers and so a ratio of 6; Llama's gated MLP has 7). Each unit
    is one FLAT plan, and the units' ledgers add up to 16 bytes per element
    of all units' padded buffers."""
    sizes = shapes.llama_7b()
    blocks = _units(sizes, per_block=True)
    linears = _units(sizes, per_block=False)
    assert len(blocks) == 33
    per_block_linear_units = (len(linears) - 1) // 32
    assert per_block_linear_units == 8  # 7 linear units + the block's norm unit
    assert per_block_linear_units - 1 == 7
    for units in (blocks, linears):
        assert sorted(n for u in units for n in u) == sorted(sizes)
        total_T, total_bytes = 0, 0
        for u in units:
            ranks = [plan_flat(u, 8, r, 1) for r in range(8)]
            total_T += ranks[0].T
            total_bytes += sum(p.persistent_bytes for p in ranks)
            assert ranks[0].T - sum(u) < 8 * 8  # padding below one granule per unit
        assert total_bytes == 16 * total_T
    # every block's unit holds the same 202,383,360 parameters; per block the
    # per-linear policy issues 7 gathers where the per-block policy issues 1
    assert {sum(u) for u in blocks[:32]} == {4 * 4096 * 4096 + 3 * 11008 * 4096 + 2 * 4096}
