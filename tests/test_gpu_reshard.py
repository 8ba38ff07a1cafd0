"""GPU <-> oracle parity of the gather into a k-way reshard slice
(reshard_after_forward as an integer: "FSDP2's parameter lifecycle...",
section "Reshard policy: pay for the memory, or pay for the communication
again").

For every divisor k of N and every rank: the plan query equals the oracle's;
the own updated shard written into the slice that holds it
(zs_gather_params_to_slice) and the kept slice assembled from its N/k source
shards (zs_gather_slice) equal the oracle's buffers bit for bit, including
64-element guard bands on both sides that must keep their sentinels. An
end-to-end case runs the fused step on all ranks and checks that every
rank's kept slice equals the same range of the FLAT gathered buffer. A world
of 300 ranks at k = 1 gathers 300 sources (more than one launch's worth).
"""
import numpy as np
import pytest

import oracle
from oracle.plan import plan_flat, reshard_slice
from gpu_util import dev16, host16

pytestmark = pytest.mark.gpu

SENT = 0x5A5A
GUARD = 64
FIELDS = ("group_size", "slice_index", "slice_off", "slice_len", "first_source", "n_sources", "owner_slice",
          "own_off", "retained_bytes")


@pytest.fixture(scope="module")
def zs():
    import torch

    import fsdp_sharded_mixed_flatten_amd as m
    torch.cuda.init()
    return m


def _divisors(n):
    return [k for k in range(1, n + 1) if n % k == 0]


def _guarded(n):
    """A sentinel-filled device buffer of n + 2*GUARD elements and its middle n."""
    buf = dev16(np.full(n + 2 * GUARD, SENT, np.uint16))
    return buf, buf[GUARD:GUARD + n]


def _check_guarded(buf, want, what):
    got = host16(buf)
    assert np.all(got[:GUARD] == SENT) and np.all(got[GUARD + want.size:] == SENT), f"{what}: guard band written"
    assert np.array_equal(got[GUARD:GUARD + want.size], want), f"{what}: differs from the oracle"


@pytest.mark.parametrize("N,numels", [(8, [100_003, 4093, 77]), (6, [55_555]), (300, [23_999])])
def test_gathers_into_reshard_slices(zs, N, numels):
    import torch
    rng = np.random.default_rng(N)
    plans = [zs.zs_shard_plan(numels, N, r, 8) for r in range(N)]
    oplans = [plan_flat(numels, N, r, 8) for r in range(N)]
    T, S = oplans[0].T, oplans[0].S
    params = [rng.integers(0, 1 << 16, S, dtype=np.uint16) for _ in range(N)]
    dparams = [dev16(p) for p in params]
    ranks = range(N) if N <= 8 else (0, 1, 150, 299)
    for k in _divisors(N):
        if N > 8 and k not in (1, 2, 300):
            continue
        for r in ranks:
            got = zs.zs_plan_reshard_slice(plans[r], k)
            want = reshard_slice(oplans[r], k)
            assert tuple(getattr(got, f) for f in FIELDS) == tuple(getattr(want, f) for f in FIELDS)
            # the own shard into the slice that holds it
            buf, view = _guarded(want.slice_len)
            zs.zs_gather_params_to_slice(plans[r], k, dparams[r], view)
            o = np.full(want.slice_len, SENT, np.uint16)
            oracle.gather_to_slice(params[r], want.own_off, o)
            torch.cuda.synchronize()
            _check_guarded(buf, o, f"N={N} k={k} r={r} own shard")
            # the kept slice from its sources
            buf, view = _guarded(want.slice_len)
            src = list(range(want.first_source, want.first_source + want.n_sources))
            zs.zs_gather_slice(plans[r], k, [dparams[q] for q in src], view)
            o = np.full(want.slice_len, SENT, np.uint16)
            oracle.gather_slice([params[q] for q in src], o)
            torch.cuda.synchronize()
            _check_guarded(buf, o, f"N={N} k={k} r={r} kept slice")


def test_fused_step_then_kept_slices_equal_the_flat_gathered_buffer(zs):
    """All 8 ranks run the fused step (bf16 param written); each rank's kept
    slice for k = 1, 2, 4, 8 assembled from the updated shards equals the same
    range of the FLAT gathered buffer the 8 ranks' gathers build, and the
    oracle's step."""
    import torch

    import synth
    numels, N, seed = [70_001, 999], 8, 77
    plans = [zs.zs_shard_plan(numels, N, r, 8) for r in range(N)]
    op = plan_flat(numels, N, 0, 8)
    T, S = op.T, op.S
    pad = np.frombuffer(bytes(op.padding_mask_full()), dtype=np.uint8).astype(bool)
    master0 = synth.cpu_f32(T, 0, synth.spec(seed, synth.STREAM_MASTER, 0, 0.02))
    master0[pad] = 0
    cs = [synth.cpu_bf16(T, 0, synth.spec(seed, synth.STREAM_CONTRIB + q, 1, 1e-3)) for q in range(N)]
    for c in cs:
        c[pad] = 0
    hp = zs.AdamWHParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)
    full = dev16(np.full(T, SENT, np.uint16))
    params = []
    o_full = np.full(T, SENT, np.uint16)
    for r in range(N):
        sl = slice(r * S, (r + 1) * S)
        master = torch.from_numpy(master0[sl].copy()).cuda()
        m, v = torch.zeros(S, device="cuda"), torch.zeros(S, device="cuda")
        p = torch.empty(S, dtype=torch.int16, device="cuda")
        zs.zs_fused_shard_step(plans[r], hp, [dev16(c[sl]) for c in cs], master, m, v, param=p, full=full)
        params.append(p)
        g, om, ov, pp = np.zeros(S, np.uint16), np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.uint16)
        oracle.shard_step(oracle.HParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, 1),
                          [c[sl].copy() for c in cs], g, master0[sl].copy(), om, ov, pp, o_full, r)
    torch.cuda.synchronize()
    h_full = host16(full)
    assert np.array_equal(h_full, o_full)
    for k in (1, 2, 4, 8):
        for r in range(N):
            s = zs.zs_plan_reshard_slice(plans[r], k)
            kept = dev16(np.full(s.slice_len, SENT, np.uint16))
            zs.zs_gather_slice(plans[r], k, params[s.first_source:s.first_source + s.n_sources], kept)
            torch.cuda.synchronize()
            assert np.array_equal(host16(kept), h_full[s.slice_off:s.slice_off + s.slice_len]), (k, r)
