"""The Python binding refuses operands that would hand a kernel a host
pointer or an out-of-range row count, before anything is launched."""

import numpy as np
import pytest

from helpers import to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nrc():
    import norm_rope_cache_amd as m

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m._load()
    return m


def _store_operands(L=2, T=8, H=8, nb=4, bs=16):
    from norm_rope_cache_amd import synth

    kv = to_dev(synth.normal_bf16(51, (L, T, 2 * H * 64)))
    pos = torch.arange(T, dtype=torch.int64)
    slots = torch.arange(T, dtype=torch.int64)
    cs = to_dev(synth.rope_table(64))
    caches = to_dev(synth.random_bits_u16(52, (L, nb, H, bs, 128)))
    return kv, pos, slots, cs, caches, H


def test_store_refuses_host_slots_positions_and_long_rows(nrc):
    kv, pos, slots, cs, caches, H = _store_operands()
    before = to_host(caches)
    L = kv.shape[0]
    cases = {
        "host slots (shared)": dict(positions=pos.cuda(), slots=slots),
        "host slots (stacked)": dict(positions=pos.cuda(), slots=slots.expand(L, -1).contiguous()),
        "host slots (list)": dict(positions=pos.cuda(), slots=[slots, slots]),
        "host positions": dict(positions=pos, slots=slots.cuda()),
        "rows beyond the mapping": dict(positions=pos.cuda(), slots=slots[:5].cuda(), rows=6),
        "negative rows": dict(positions=pos.cuda(), slots=slots.cuda(), rows=-1),
    }
    for what, kw in cases.items():
        with pytest.raises(ValueError):
            nrc.context_kv_store(kv, kw["positions"], kw["slots"], cs, caches, H, rows=kw.get("rows"))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(caches), before), "a refused call wrote the cache"


def test_project_store_refuses_host_operands_and_long_rows(nrc):
    """The one-call projection + store checks the store's operands before
    anything runs: nothing written to kv or the caches."""
    from norm_rope_cache_amd import synth

    kv, pos, slots, cs, caches, H = _store_operands()
    L, T = kv.shape[0], kv.shape[1]
    normed = to_dev(synth.normal_bf16(63, (L, T, 8192)))
    w = to_dev(synth.normal_bf16(64, (L, 8192, 2 * H * 64), std=0.02))
    out = torch.zeros_like(kv)
    before = to_host(caches)
    long_slots = torch.arange(T + 3, dtype=torch.int64)
    cases = {
        "host slots": dict(positions=pos.cuda(), slots=slots),
        "host positions": dict(positions=pos, slots=slots.cuda()),
        "rows beyond the mapping": dict(positions=pos.cuda(), slots=slots[:5].cuda(), rows=6),
        "rows beyond T": dict(positions=long_slots.cuda(), slots=long_slots.cuda(), rows=T + 1),
    }
    for what, kw in cases.items():
        with pytest.raises(ValueError):
            nrc.context_kv_project_store(normed, w, kw["positions"], kw["slots"], cs, caches, rows=kw.get("rows"),
                                         out=out)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(caches), before), "a refused call wrote the cache"
    assert not bool(out.view(torch.int16).any()), "a refused call wrote kv"


def test_store_ex_refuses_host_slots_and_positions(nrc):
    kv, pos, slots, cs, caches, H = _store_operands()
    before = to_host(caches)
    views = [caches[0], caches[1]]
    with pytest.raises(ValueError):
        nrc.context_kv_store_ex(kv, pos.cuda(), [slots, slots.cuda()], cs, views, H)
    with pytest.raises(ValueError):
        nrc.context_kv_store_ex(kv, pos, [slots.cuda(), slots.cuda()], cs, views, H)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(caches), before), "a refused call wrote the cache"


def test_fused_projection_refuses_a_host_scale(nrc):
    from norm_rope_cache_amd import synth

    T, L, N = 4, 1, 128
    h = to_dev(synth.normal_bf16(61, (T, 8192)))
    w = to_dev(synth.normal_bf16(62, (L, 8192, N), std=0.02))
    out = torch.zeros((L, T, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        nrc.context_kv_project_fused(h, torch.ones(T, dtype=torch.float32), None, w, out=out)
    with pytest.raises(ValueError):
        nrc.context_hidden_norm(h, None, None, L, r=torch.empty(T, dtype=torch.float32))
    torch.cuda.synchronize()
    assert not bool(out.view(torch.int16).any()), "a refused call wrote the output"


def test_shared_slot_mapping_equals_stacked_copies(nrc):
    """One [rows] mapping handed to every layer writes what L identical
    copies write."""
    from norm_rope_cache_amd import synth

    kv, pos, _, cs, caches, H = _store_operands(L=3, T=40, nb=8)
    slots = torch.from_numpy(synth.permutation(7, 8 * 16)[:40].copy()).cuda()
    slots[5] = -1
    a, b = caches.clone(), caches.clone()
    nrc.context_kv_store(kv, torch.arange(40, dtype=torch.int64, device="cuda"), slots, to_dev(synth.rope_table(64)),
                         a, H)
    nrc.context_kv_store(kv, torch.arange(40, dtype=torch.int64, device="cuda"), slots.expand(3, -1).contiguous(),
                         to_dev(synth.rope_table(64)), b, H)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(a), to_host(b))
    assert not np.array_equal(to_host(a), to_host(caches))


def test_norm_bindings_refuse_misshaped_and_host_operands(nrc):
    """Every operand the norm kernels read or write is checked for shape and
    device before a launch: a short weight or output would otherwise be read
    or written past its end."""
    from norm_rope_cache_amd import synth

    T, L = 3, 2
    x = to_dev(synth.normal_bf16(71, (T, 8192)))
    hw = to_dev(synth.normal_bf16(72, (8192,), mean=1.0, std=0.1))
    pw = to_dev(synth.normal_bf16(73, (L, 8192), mean=1.0, std=0.1))
    h = torch.zeros((T, 8192), dtype=torch.bfloat16, device="cuda")
    r = torch.zeros((T,), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        nrc.context_hidden_norm(x, hw[:4096], pw, L, h=h, r=r)
    with pytest.raises((TypeError, ValueError)):
        nrc.context_hidden_norm(x, hw.cpu(), pw, L, h=h, r=r)
    with pytest.raises(ValueError):
        nrc.context_hidden_norm(x[0], hw, pw, L, h=h, r=r)
    out = torch.zeros((L, T, 8192), dtype=torch.bfloat16, device="cuda")
    with pytest.raises((TypeError, ValueError)):
        nrc.context_norms(x, hw, pw, L, out=out.cpu())
    with pytest.raises((TypeError, ValueError)):
        nrc.context_norms_ex(x, hw.float().cpu(), pw, L, out=out)

    branch = to_dev(synth.normal_bf16(74, (T, 8192)))
    s_in = torch.zeros((T, 8192), dtype=torch.float32, device="cuda")
    alpha = torch.ones(8192, dtype=torch.float32, device="cuda")
    beta = torch.ones(8192, dtype=torch.float32, device="cuda")
    b_out = torch.zeros((T, 8192), dtype=torch.bfloat16, device="cuda")
    s_out = torch.zeros((T, 8192), dtype=torch.float32, device="cuda")
    cases = {
        "short out": dict(out=b_out[:1]),
        "float32 out": dict(out=s_out),
        "short stream_out": dict(out=b_out, stream_out=s_out[:1]),
        "bf16 stream_out": dict(out=b_out, stream_out=b_out),
        "host stream_out": dict(out=b_out, stream_out=s_out.cpu()),
        "host alpha": dict(out=b_out, alpha=alpha.cpu()),
    }
    for what, kw in cases.items():
        a = kw.pop("alpha", alpha)
        with pytest.raises((TypeError, ValueError)):
            nrc.draft_boundary(branch, s_in, a, beta, hw, hw, **kw)
    torch.cuda.synchronize()
    for t in (h, r, out, b_out, s_out):
        assert not bool(t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).any()), \
            "a refused call wrote an output"
