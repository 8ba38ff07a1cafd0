"""The library's host AdamW (the CPU side of the offloaded step) against the
oracle, on the CPU: bit-identical master/m/v and bf16 parameters over several
steps, for several thread counts and ragged lengths, including non-finite
and subnormal gradients. It runs without a GPU: the host step touches no
device memory."""
import numpy as np
import pytest

import oracle
import synth
from conftest import import_zs


@pytest.fixture(scope="module")
def zs():
    return import_zs()


def _grads(n, t, seed):
    g = synth.cpu_bf16(n, 0, synth.spec(seed, synth.STREAM_CONTRIB, t, 1e-3, 2**62, 0.1, 0.001, 0.01))
    g[::997] = 0x7FC0  # NaN
    g[5::1009] = 0xFF80  # -inf
    g[7::1013] = 0x0003  # subnormal
    return g


@pytest.mark.parametrize("n,threads", [(1, 1), (37, 3), (100_003, 1), (100_003, 8), (262_144, 16)])
def test_host_adamw_equals_oracle(zs, n, threads):
    master0 = synth.cpu_f32(n, 0, synth.spec(3, synth.STREAM_MASTER, 0, 0.02, n))
    a = dict(master=master0.copy(), m=np.zeros(n, np.float32), v=np.zeros(n, np.float32), p=np.zeros(n, np.uint16))
    b = {k: x.copy() for k, x in a.items()}
    for t in (1, 2, 3):
        g = _grads(n, t, 4)
        hp = zs.AdamWHParams(lr=3e-4, weight_decay=0.05, step=t)
        zs.zs_host_adamw_step(hp, g, a["master"], a["m"], a["v"], a["p"], n_threads=threads)
        oracle.adamw(oracle.HParams(lr=3e-4, weight_decay=0.05, step=t), g, b["master"], b["m"], b["v"], b["p"])
        for k in a:
            assert a[k].tobytes() == b[k].tobytes() or _same_up_to_nan(a[k], b[k]), (t, k)


def _same_up_to_nan(x, y):
    """Bytes equal except NaN payload/sign (the element's NaN-ness must agree)."""
    if x.dtype == np.uint16:
        nx = ((x & 0x7F80) == 0x7F80) & ((x & 0x7F) != 0)
        ny = ((y & 0x7F80) == 0x7F80) & ((y & 0x7F) != 0)
    else:
        nx, ny = np.isnan(x), np.isnan(y)
    return np.array_equal(nx, ny) and np.array_equal(x[~nx], y[~ny])


def test_host_adamw_without_param_and_torch_tensors(zs):
    import torch
    n = 4096
    g = _grads(n, 1, 9)
    st = [torch.from_numpy(synth.cpu_f32(n, 0, synth.spec(9, synth.STREAM_MASTER, 0, 0.02, n))),
          torch.zeros(n), torch.zeros(n)]
    ref = [x.numpy().copy() for x in st] + [np.zeros(n, np.uint16)]
    zs.zs_host_adamw_step(zs.AdamWHParams(step=1), torch.from_numpy(g.view(np.int16)), *st, n_threads=2)
    oracle.adamw(oracle.HParams(step=1), g, *ref)
    for x, y in zip(st, ref[:3]):
        assert _same_up_to_nan(x.numpy(), y)


def test_host_adamw_rejects_bad_arguments(zs):
    n = 64
    a = [np.zeros(n, np.float32) for _ in range(3)]
    g = np.zeros(n, np.uint16)
    with pytest.raises(zs.ZsError):
        zs.zs_host_adamw_step(zs.AdamWHParams(step=0), g, *a)
    with pytest.raises(zs.ZsError):
        zs.zs_host_adamw_step(zs.AdamWHParams(), g, *a, n_threads=0)
    with pytest.raises(ValueError):
        zs.zs_host_adamw_step(zs.AdamWHParams(), g.astype(np.float32), *a)
    L = zs.lib()
    assert L.zs_host_adamw_step(zs.AdamWHParams(), None, a[0].ctypes.data, a[1].ctypes.data, a[2].ctypes.data,
                                None, n, 1) == zs.ZS_EINVAL
