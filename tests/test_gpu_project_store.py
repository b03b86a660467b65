"""The one-call projection + store (nrc_context_kv_project_store) against the
two calls it stands for - page "...runtime.draft", ContextKV: _project, then
store on the k/v views of the projection's own output - and against the
oracle's store run on the GPU's own kv: kv and every cache cell bit for bit.
Split shapes (small T: the store's kernel adds the slices) and unsplit ones
(the one-pass projection, then the store), more than 8 layers, ragged row
counts, negative slots, RoPE off, block sizes that are not powers of two,
both weight layouts."""

import numpy as np
import pytest

from helpers import assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


# (L, T, H, block_size, num_blocks, inserted rows, RoPE, slot form, weight layout)
CASES = [
    (4, 512, 8, 16, 64, 512, True, "shared", "dn"),      # the prefill shape: eight slices
    (2, 16, 2, 7, 5, 16, True, "per-layer", "dn"),       # sixteen slices of 128 x 128 tiles
    (10, 40, 2, 24, 9, 30, False, "per-layer", "dn"),    # two launches of layers, rows < T, RoPE off
    (1, 130, 1, 1, 300, 130, True, "shared", "dn"),      # one head, ragged 128 x 128 tiles
    (3, 700, 4, 16, 64, 650, True, "shared", "nd"),      # [L, N, D] weights
    (2, 300, 16, 5, 70, 300, True, "per-layer", "dn"),   # sixteen heads
    (4, 4096, 8, 16, 512, 4096, True, "shared", "dn"),   # no split: one pass, then the store
]


@pytest.mark.parametrize("L,T,H,bs,nb,rows,rope,slot_form,layout", CASES)
def test_project_store_matches_the_two_calls(nrc, oracle, L, T, H, bs, nb, rows, rope, slot_form, layout):
    from norm_rope_cache_amd import synth

    N = 2 * H * 64
    lib = nrc._load()
    need = lib.nrc_context_kv_project_workspace_bytes(L, T, 8192, N)
    _say(f"project+store L={L} T={T} H={H} bs={bs} rows={rows} rope={rope} {slot_form} {layout} "
         f"workspace={need}")
    assert (need > 0) == (T < 4096), "the cases above split exactly when T is small"
    rng = np.random.default_rng(L * 7919 + T)
    A = synth.normal_bf16(7100 + T, (L, T, 8192))
    B = synth.normal_bf16(7200 + N, (L, 8192, N), std=0.02)
    if slot_form == "shared":
        slots = rng.permutation(nb * bs)[:T].astype(np.int64)
        slots[rng.random(T) < 0.1] = -1
        slots_h = np.broadcast_to(slots, (L, T))
        slots_d = to_dev(slots)
    else:
        slots_h = np.stack([rng.permutation(nb * bs)[:T] for _ in range(L)]).astype(np.int64)
        slots_h[rng.random((L, T)) < 0.2] = -1
        slots_d = [to_dev(s) for s in slots_h]
    positions = rng.integers(0, 512, T).astype(np.int64)
    tab = synth.rope_table(512) if rope else None
    caches = synth.random_bits_u16(7300 + L, (L, nb, H, bs, 128))
    Ad = to_dev(A)
    Bd = to_dev(B if layout == "dn" else np.ascontiguousarray(np.swapaxes(B, 1, 2)))
    pos_d = to_dev(positions)
    tab_d = None if tab is None else to_dev(tab)

    # the two calls
    c_two = to_dev(caches)
    kv_two = nrc.context_kv_project(Ad, Bd, w_layout=layout)
    nrc.context_kv_store(kv_two, pos_d, slots_d, tab_d, c_two, H, 1e-6, rows=rows)
    # the one call, twice (the second over the first's caches: same cells, same bits)
    c_one = to_dev(caches)
    kv_one = torch.full((L, T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    for rep in range(2):
        out = nrc.context_kv_project_store(Ad, Bd, pos_d, slots_d, tab_d, c_one, 1e-6, rows=rows, out=kv_one,
                                           w_layout=layout)
        assert out is kv_one
        torch.cuda.synchronize()
        kv_h = to_host(kv_one)
        assert_bits_equal(kv_h, to_host(kv_two), f"kv, call {rep}")
        assert_bits_equal(to_host(c_one), to_host(c_two), f"caches, call {rep}")
    # the oracle's store of the GPU's own projection output
    want = caches.copy()
    oracle.context_kv_store(kv_h, H, positions[:rows], np.ascontiguousarray(slots_h[:, :rows]), tab, want, bs, 1e-6)
    assert_bits_equal(to_host(c_one), want, "caches vs the oracle's store of the GPU's kv")


def test_project_store_no_rows_is_the_projection(nrc):
    """rows == 0: the projection alone (kv written, caches untouched)."""
    from norm_rope_cache_amd import synth

    L, T, H = 2, 300, 4
    N = 2 * H * 64
    Ad = to_dev(synth.normal_bf16(7400, (L, T, 8192)))
    Bd = to_dev(synth.normal_bf16(7401, (L, 8192, N), std=0.02))
    caches = synth.random_bits_u16(7402, (L, 20, H, 16, 128))
    c = to_dev(caches)
    slots = to_dev(np.arange(T, dtype=np.int64))
    kv = nrc.context_kv_project_store(Ad, Bd, None, slots, None, c, rows=0)
    torch.cuda.synchronize()
    assert_bits_equal(to_host(kv), to_host(nrc.context_kv_project(Ad, Bd)), "kv")
    assert_bits_equal(to_host(c), caches, "caches untouched")


def test_project_store_special_values(nrc):
    """Rows whose projection sums are NaN, +-Inf or overflow (normed rows with
    Inf, NaN or values near the bf16 maximum) take the same path through the
    store kernel that adds the slices as through the adding kernel and the
    store: the same kv and cache bits (split shape, RoPE on and off)."""
    from norm_rope_cache_amd import synth

    L, T, H, bs, nb = 2, 300, 2, 16, 32
    N = 2 * H * 64
    A = synth.normal_bf16(7500, (L, T, 8192))
    A[0, 3, 100] = 0x7F80          # +Inf
    A[1, 7, 5] = 0xFF80            # -Inf
    A[0, 11, 9] = 0x7FC1           # NaN
    A[1, 13, :64] = 0x7F7F         # bf16 max: sums overflow
    A[0, 17] = 0x8000              # an all -0.0 row
    B = synth.normal_bf16(7501, (L, 8192, N), std=0.02)
    rng = np.random.default_rng(7502)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    pos = rng.integers(0, 256, T).astype(np.int64)
    caches = synth.random_bits_u16(7503, (L, nb, H, bs, 128))
    Ad, Bd = to_dev(A), to_dev(B)
    need = nrc._load().nrc_context_kv_project_workspace_bytes(L, T, 8192, N)
    assert need > 0, "the shape must split"
    for rope in (True, False):
        _say(f"project+store special values rope={rope}")
        tab = to_dev(synth.rope_table(256)) if rope else None
        c_two, c_one = to_dev(caches), to_dev(caches)
        kv_two = nrc.context_kv_project(Ad, Bd)
        nrc.context_kv_store(kv_two, to_dev(pos), to_dev(slots), tab, c_two, H)
        kv_one = nrc.context_kv_project_store(Ad, Bd, to_dev(pos), to_dev(slots), tab, c_one)
        torch.cuda.synchronize()
        kv_h = to_host(kv_one)
        assert_bits_equal(kv_h, to_host(kv_two), f"kv rope={rope}")
        assert_bits_equal(to_host(c_one), to_host(c_two), f"caches rope={rope}")
        f = (kv_h.astype(np.uint32) << 16).view(np.float32)
        assert np.isnan(f).any() and np.isinf(f).any(), "the inputs must reach NaN and Inf sums"
