"""Pins of the plan variants: a persistence threshold (small tensors
replicated, not sharded) and per-tensor hyperparameter groups.

* [P2]'s section 7 example: a 768-element layer norm over 64 ranks is a
  12-element shard when sharded; under a threshold of 1e5 (the value the page
  suggests) it stays whole on every rank.
* coverage: sharded tensors are owned exactly once over the ranks, replicated
  ones by every rank; the ledger counts replicated tensors on every rank.
* groups: AdamW with a zero-decay group equals PyTorch's AdamW with two
  parameter groups (float64).
"""
import json
import os
import random

import numpy as np
import pytest
import torch

import oracle
from oracle.plan import plan_per_tensor
from synth import shapes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ledger_numbers.json")))


def test_norm_768_stays_replicated_under_threshold():
    g = GOLD["norm_768_over_64"]
    sharded = plan_per_tensor([g["numel"]], g["world"], 5)
    assert sharded.S == 16  # 12 real elements' worth of shard, 16-element granule
    kept = plan_per_tensor([g["numel"]], g["world"], 5, persist_below=100_000)
    (pc,) = kept.pieces
    assert (pc.own_lo, pc.own_hi, pc.real_hi) == (0, 768, 768) and kept.S == 768
    assert kept.persistent_bytes == 16 * 768


def test_llama7b_norms_replicated():
    sizes = shapes.llama_7b()
    p = plan_per_tensor(sizes, 8, 3, persist_below=100_000)
    repl = [pc for pc, n in zip(p.pieces, sizes) if n < 100_000]
    assert len(repl) == 65 and all(pc.own_hi - pc.own_lo == 4096 for pc in repl)
    sharded_S = sum((n + 63) // 64 * 64 // 8 for n in sizes if n >= 100_000)
    assert p.S == sharded_S + 65 * 4096
    assert p.persistent_bytes == 16 * p.S


@pytest.mark.parametrize("seed", range(12))
def test_coverage_with_threshold(seed):
    rnd = random.Random(seed)
    numels = [rnd.choice([1, 7, 64, 100, 768, 1000, 5000]) for _ in range(rnd.randint(1, 10))]
    world = rnd.choice([1, 2, 3, 4, 8])
    thr = rnd.choice([0, 8, 100, 1000, 10_000])
    owners = {}
    written = {}  # gathered-buffer position -> ranks whose piece writes it
    for r in range(world):
        p = plan_per_tensor(numels, world, r, thr)
        assert p.S % 8 == 0 and p.persistent_bytes == 16 * p.S
        for pc in p.pieces:
            for k in range(pc.real_lo, pc.real_hi):
                owners.setdefault((pc.tensor, k), []).append(r)
            assert p.offsets[pc.tensor] <= pc.full_off
            assert pc.full_off + pc.own_hi - pc.own_lo <= p.offsets[pc.tensor] + p.padded[pc.tensor]
            for x in range(pc.full_off, pc.full_off + pc.own_hi - pc.own_lo):
                written.setdefault(x, []).append(r)
    # every position of the gathered buffer is written: by every rank for a
    # replicated tensor, by exactly one rank otherwise
    assert sorted(written) == list(range(p.T))
    for i, (o, Ti) in enumerate(zip(p.offsets, p.padded)):
        for x in range(o, o + Ti):
            assert written[x] == (list(range(world)) if numels[i] < thr else written[x][:1]), (i, x)
    for (i, k), rs in owners.items():
        if numels[i] < thr:
            assert rs == list(range(world))
        else:
            assert len(rs) == 1
    assert sum(1 for (i, _k) in owners) == sum(numels)


def test_groups_against_torch_param_groups():
    rng = np.random.default_rng(9)
    sizes = [4096, 64, 2048]  # weight, bias-like, weight
    decay_group = [True, False, True]
    lr, wd, steps = 3e-3, 0.3, 6
    masters = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    st = [[mm, np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)] for mm, n in zip(masters, sizes)]
    ws = [torch.nn.Parameter(torch.from_numpy(mm.astype(np.float64))) for mm in masters]
    opt = torch.optim.AdamW([{"params": [w for w, d in zip(ws, decay_group) if d], "weight_decay": wd},
                             {"params": [w for w, d in zip(ws, decay_group) if not d], "weight_decay": 0.0}],
                            lr=lr, betas=(0.9, 0.95), eps=1e-8, foreach=False)
    for t in range(1, steps + 1):
        for i, n in enumerate(sizes):
            x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
            g = (x.view(np.uint32) >> 16).astype(np.uint16)
            hp = oracle.HParams(lr=lr, weight_decay=wd if decay_group[i] else 0.0, step=t)
            g_arr = g
            oracle.adamw(hp, g_arr, *st[i])
            ws[i].grad = torch.from_numpy(oracle.bf16_to_f32(g).astype(np.float64))
        opt.step()
        for i in range(len(sizes)):
            ref = ws[i].detach().numpy()
            tol = 4 * t * 2.0**-24 * (np.abs(ref) + lr) + lr * 1e-6
            assert np.all(np.abs(st[i][0] - ref) <= tol)
    # the zero-decay group is exactly AdamW without decay: decay factor 1
    assert oracle.adamw_coef(lr, 0.9, 0.95, 1e-8, 0.0, 1)[6] == 1.0
