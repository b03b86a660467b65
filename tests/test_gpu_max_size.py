"""The chain at its largest single-call size: L = 8 draft layers, T = 131072
rows, H = 16 heads (N = 2048), so the stacked norms (17 GB), kv (4.3 GB)
and the caches (4.3 GB) all put element offsets past 2^31 and byte offsets
past 2^32 in every kernel. The rows repeat a 512-row seeded base (built on
the device), so the whole output is checked: every row of the norms and of
kv equals its base row's bit for bit; the base rows match the oracle (norms
bit-exact, projection within tolerance); the cache cells of sampled rows
equal the oracle's store of the GPU's own kv for those rows, and every cell
that no row writes is untouched."""

import numpy as np
import pytest

from helpers import assert_bits_equal, projection_tolerance_ok, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

L, T, H, D, BASE = 8, 131072, 16, 8192, 512
N = 2 * H * 64
BS, NB = 64, 2048  # 131072 slots


@pytest.fixture(scope="module")
def nrc():
    import norm_rope_cache_amd as m

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m._load()
    return m


@pytest.fixture(scope="module")
def oracle():
    import oracle as o

    o.lib()
    return o


def _say(*a):
    print(*a, flush=True)


def _periodic(t, what):
    """Every BASE-row block of dim 1 equals the first, bit for bit (a layer
    at a time, to bound the comparison's memory)."""
    v = t.view(torch.int16)
    for l in range(v.shape[0]):
        blocks = v[l].view(T // BASE, BASE, v.shape[2])
        bad = int((blocks != blocks[:1]).any(dim=2).sum().item())
        assert bad == 0, f"{what}, layer {l}: {bad} rows differ from their base row"


def test_chain_at_the_largest_size(nrc, oracle):
    from norm_rope_cache_amd import synth

    _say(f"max size: L={L} T={T} H={H} N={N}")
    base = synth.normal_bf16(8100, (BASE, D))
    hw = synth.normal_bf16(8101, (D,), mean=1.0, std=0.1)
    pw = synth.normal_bf16(8102, (L, D), mean=1.0, std=0.1)
    w = synth.normal_bf16(8103, (L, D, N), std=0.02)
    rng = np.random.default_rng(8104)
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)
    slots[rng.random(T) < 0.1] = -1
    positions = rng.integers(0, 131072, T).astype(np.int64)
    tab = synth.rope_table(131072)
    caches0 = synth.random_bits_u16(8105, (L, NB, H, BS, 128))

    x = to_dev(base).repeat(T // BASE, 1)
    normed = nrc.context_norms(x, to_dev(hw), to_dev(pw), L)
    del x
    torch.cuda.synchronize()
    _periodic(normed, "norms")
    want_n = oracle.context_norms(base, hw, pw, L)
    assert_bits_equal(to_host(normed[:, :BASE]), want_n, "norms of the base rows")
    _say("norms ok")

    kv = nrc.context_kv_project(normed, to_dev(w))
    del normed
    torch.cuda.synchronize()
    _periodic(kv, "kv")
    rows = np.arange(0, BASE, 8)
    kv_rows = to_host(kv[:, torch.as_tensor(rows, device=kv.device)])
    ok, msg = projection_tolerance_ok(kv_rows, oracle.kv_project(np.ascontiguousarray(want_n[:, rows]), w))
    assert ok, msg
    _say("projection ok")

    caches = to_dev(caches0)
    nrc.context_kv_store(kv, to_dev(positions), to_dev(slots), to_dev(tab), caches, H)
    torch.cuda.synchronize()
    got = to_host(caches)
    del caches
    # sampled rows (first, last, every 997th, and negative-slot rows among them)
    sample = np.unique(np.concatenate([[0, T - 1], np.arange(0, T, 997)]))
    kv_s = to_host(kv[:, torch.as_tensor(sample, device=kv.device)])
    want = caches0.copy()
    oracle.context_kv_store(kv_s, H, positions[sample], np.ascontiguousarray(np.broadcast_to(slots[sample], (L, sample.size))),
                            tab, want, BS)
    live = slots[sample][slots[sample] >= 0]
    blk, page = live // BS, live % BS
    assert_bits_equal(got[:, blk, :, page], want[:, blk, :, page], "cache cells of the sampled rows")
    # every cell no row writes is untouched
    written = np.zeros(NB * BS, dtype=bool)
    written[slots[slots >= 0]] = True
    free = np.flatnonzero(~written)
    assert free.size > 0
    assert_bits_equal(got[:, free // BS, :, free % BS], caches0[:, free // BS, :, free % BS], "cells no row writes")
    _say(f"store ok: {live.size} sampled rows, {free.size} free slots")
