"""One library used from several host threads at once, each thread on its own
HIP stream.

Plans are immutable and shared across threads; the error text of the last
failed call is per thread; the registry of bound multi-tensor workspaces is
shared under a lock. Each thread runs its own steps (flat bucketed, flat
fused, multi-tensor unfused and fused) on its own state, binds and unbinds
scratch workspaces in a loop, and makes failing calls whose messages must be
its own. Afterwards every thread's state must equal the oracle's exactly, as
when the runs execute alone.
"""
import threading

import pytest

from test_gpu_parity import FlatRun, MultiRun, _small_model

pytestmark = pytest.mark.gpu

THREADS = 4
STEPS = 3


@pytest.fixture(scope="module")
def zs():
    import torch

    import fsdp_sharded_mixed_flatten_amd as m
    torch.cuda.init()
    return m


def _hp(zs):
    return zs.AdamWHParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)


def test_threads_with_own_streams(zs):
    import torch
    hp = _hp(zs)
    # flat runs of the same rank share one plan object; seeds differ
    flat = [FlatRun(zs, [1_000_003], 4, 1, 1, STEPS, 500 + i, hp, bucket=65_536, fused=bool(i % 2))
            for i in range(THREADS)]
    shared = flat[0].plan
    for run in flat:
        run.plan = shared
    multi = [MultiRun(zs, _small_model(), 8, 3, STEPS, 600 + i, hp) for i in range(THREADS)]
    scratch = []
    for run in multi:
        nbytes = zs.zs_multi_workspace_bytes(run.plan, run.n_contribs)
        scratch.append([torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)])
    torch.cuda.synchronize()
    barrier = threading.Barrier(THREADS)
    errors = []

    def work(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for t in range(1, STEPS + 1):
                    flat[i].step(t)
                    multi[i].step(t, fused=bool(t % 2))
                    # bind and unbind scratch workspaces while the other threads run
                    for ws in scratch[i]:
                        zs.zs_multi_bind(multi[i].plan, multi[i].pieces, multi[i].dcontribs[t], ws)
                    for ws in scratch[i]:
                        zs.zs_multi_unbind(ws)
                    # a failing call: the message must name this thread's arguments
                    bad_rank = 1000 + 10 * i + t
                    barrier.wait(timeout=60)
                    with pytest.raises(zs.ZsError) as e:
                        zs.zs_shard_plan([16], 4, bad_rank)
                    barrier.wait(timeout=60)
                    assert f"rank = {bad_rank}" in zs.zs_last_error(), zs.zs_last_error()
                    assert f"rank = {bad_rank}" in e.value.message
                stream.synchronize()
        except BaseException as exc:  # re-raised in the main thread
            errors.append((i, exc))
            barrier.abort()

    threads = [threading.Thread(target=work, args=(i,)) for i in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
        assert not th.is_alive(), "a worker thread did not finish"
    if errors:
        i, exc = errors[0]
        raise AssertionError(f"thread {i} failed: {exc!r}") from exc
    torch.cuda.synchronize()
    for run in flat:
        run.check()
    for run in multi:
        run.check()
