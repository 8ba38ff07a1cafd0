"""zs_grad_stats_noalloc, the squared-norm and non-finite check without a
workspace (its partials live in the library's static per-GPU array), against
zs_grad_stats with a caller workspace: identical bits on consecutive calls
of different sizes, the later calls smaller than the first, so partials a
previous call left in the shared array must never be read; both against the
oracle's double sum within relative 1e-12."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zs():
    import torch

    import fsdp_sharded_mixed_flatten_amd as m
    torch.cuda.init()
    return m


def _acc(n, seed, nan_at=None):
    a = synth.cpu_f32(n, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 3e-3))
    if nan_at is not None:
        a[nan_at] = np.float32(np.nan)
    return a


def _both(zs, plan, acc_h, divisor):
    import torch
    acc = dev32(acc_h)
    out = torch.full((2,), -1.0, dtype=torch.float64, device="cuda")
    flags = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(zs.zs_grad_stats_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    zs.zs_grad_stats(plan, acc, divisor, out[0:1], flags[0:1], ws)
    zs.zs_grad_stats_noalloc(plan, acc, divisor, out[1:2], flags[1:2])
    torch.cuda.synchronize()
    s = out.cpu().numpy()
    f = flags.cpu().numpy()
    return s, f


def test_noalloc_equals_workspace_call_on_shrinking_calls(zs):
    cases = [
        # (numels, world, rank, divisor, nan position or None)
        ([3_000_011, 4093], 4, 1, 4.0, None),       # 184 blocks of partials
        ([100_003], 2, 0, 1.0, 33_333),              # 13 blocks, a NaN: the flag must be set
        ([5_000], 4, 3, 2.0, None),                  # 1 block: the flag must not stick
    ]
    for numels, N, r, divisor, nan_at in cases:
        plan = zs.zs_shard_plan(numels, N, r, 1)
        S = plan.shard_numel
        acc_h = _acc(S, 1000 + S, nan_at)
        s, f = _both(zs, plan, acc_h, divisor)
        assert s.view(np.uint64)[0] == s.view(np.uint64)[1] or (np.isnan(s[0]) and np.isnan(s[1])), \
            f"S={S}: workspace {s[0]!r} != static scratch {s[1]!r}"
        assert f[0] == f[1] == (1 if nan_at is not None else 0), f"S={S}: flags {f}"
        o_s, o_f = oracle.grad_sumsq(acc_h, divisor)
        assert o_f == f[1]
        if nan_at is None:
            assert abs(s[1] - o_s) <= 1e-12 * o_s, (s[1], o_s)


def test_noalloc_full_width_then_smaller(zs):
    """The largest shard the static array serves (a full array of partials),
    then a smaller one."""
    import torch
    S_max = zs.GRAD_STATS_NOALLOC_MAX_ELEMS
    free, _ = torch.cuda.mem_get_info()
    if free < S_max * 4 * 2 + (4 << 30):
        pytest.skip("needs ~15 GiB of free device memory")
    plan = zs.zs_shard_plan([S_max], 1, 0, 1)
    assert plan.shard_numel == S_max
    acc = torch.empty(S_max, dtype=torch.float32, device="cuda")
    synth.gpu_f32(acc, 0, synth.spec(77, synth.STREAM_MASTER, 0, 1e-3))
    out = torch.full((2,), -1.0, dtype=torch.float64, device="cuda")
    flags = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(zs.zs_grad_stats_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    zs.zs_grad_stats(plan, acc, 1.0, out[0:1], flags[0:1], ws)
    zs.zs_grad_stats_noalloc(plan, acc, 1.0, out[1:2], flags[1:2])
    torch.cuda.synchronize()
    s = out.cpu().numpy()
    assert s.view(np.uint64)[0] == s.view(np.uint64)[1]
    assert flags.cpu().tolist() == [0, 0]
    # the oracle's double sum over a sample prefix of the same values agrees
    # with a prefix call (1,000,000 elements, rank-0 plan over exactly that)
    n = 1_000_000
    plan_small = zs.zs_shard_plan([n], 1, 0, 1)
    s2, f2 = _both(zs, plan_small, acc[:n].cpu().numpy(), 1.0)
    assert s2.view(np.uint64)[0] == s2.view(np.uint64)[1] and f2.tolist() == [0, 0]
    o_s, _ = oracle.grad_sumsq(acc[:n].cpu().numpy(), 1.0)
    assert abs(s2[1] - o_s) <= 1e-12 * o_s
    del acc, ws
    torch.cuda.empty_cache()


def test_noalloc_rejects_a_shard_past_the_static_array(zs):
    plan = zs.zs_shard_plan([zs.GRAD_STATS_NOALLOC_MAX_ELEMS + 8], 1, 0, 1)
    import torch
    acc = torch.empty(16, dtype=torch.float32, device="cuda")  # never read: the call fails first
    with pytest.raises(zs.ZsError) as ei:
        zs.zs_grad_stats_noalloc(plan, acc.data_ptr(), 1.0, torch.zeros(1, dtype=torch.float64, device="cuda"),
                                 torch.zeros(1, dtype=torch.int32, device="cuda"))
    assert ei.value.status == zs.ZS_ENOMEM
