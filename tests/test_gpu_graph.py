"""The chain's calls are asynchronous on the caller's stream and capturable
into a graph, as the context page states for ContextNorms and
ContextKvStore (a call is graph-capturable): the whole chain captured once
into a HIP graph (torch.cuda.CUDAGraph) replays to the eager bits, replay
after replay, with eager work and synchronisations between the replays;
and chains issued on two explicit streams at once each give the eager
bits."""

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


def _say(msg):
    print(msg, flush=True)


class _Chain:
    """One buffer set of the chain on device: inputs, the stacked norms (or
    the fused form's h and r), kv and the caches."""

    def __init__(self, nrc, cfg, d, fused, one_call=False):
        self.nrc, self.cfg, self.d, self.fused, self.one_call = nrc, cfg, d, fused, one_call
        self.x = to_dev(d["x"])
        self.hw = None if d["hidden_w"] is None else to_dev(d["hidden_w"])
        self.pw = None if d["pre_w"] is None else to_dev(d["pre_w"])
        self.w = to_dev(d["w_kv"])
        self.pos = to_dev(d["positions"])
        self.slots = to_dev(d["slots"][0])
        self.cs = None if d["cos_sin"] is None else to_dev(d["cos_sin"])
        self.caches0 = to_dev(d["caches"])
        self.caches = self.caches0.clone()
        self.kv = torch.empty((cfg.L, cfg.T, cfg.N), dtype=torch.bfloat16, device="cuda")
        if fused:
            self.h = torch.empty((cfg.T, 8192), dtype=torch.bfloat16, device="cuda")
            self.r = torch.empty((cfg.T,), dtype=torch.float32, device="cuda")
        else:
            self.normed = torch.empty((cfg.L, cfg.T, 8192), dtype=torch.bfloat16, device="cuda")

    def run(self):
        nrc, cfg, d = self.nrc, self.cfg, self.d
        if self.one_call:
            nrc.context_norms(self.x, self.hw, self.pw, cfg.L, d["hidden_eps"], d["pre_eps"], out=self.normed)
            nrc.context_kv_project_store(self.normed, self.w, self.pos, self.slots, self.cs, self.caches,
                                         d["k_eps"], out=self.kv)
            return
        if self.fused:
            nrc.context_hidden_norm(self.x, self.hw, self.pw, cfg.L, d["hidden_eps"], d["pre_eps"], h=self.h, r=self.r)
            nrc.context_kv_project_fused(self.h, self.r, self.pw, self.w, out=self.kv)
        else:
            nrc.context_norms(self.x, self.hw, self.pw, cfg.L, d["hidden_eps"], d["pre_eps"], out=self.normed)
            nrc.context_kv_project(self.normed, self.w, out=self.kv)
        nrc.context_kv_store(self.kv, self.pos, self.slots, self.cs, self.caches, cfg.H, d["k_eps"])

    def reset(self):
        self.caches.copy_(self.caches0)
        self.kv.view(torch.int16).fill_(-1)


@pytest.mark.parametrize("name,fused,one_call", [("tiny", False, False), ("prefill", False, False),
                                                 ("prefill", True, False), ("weightless", False, False),
                                                 ("tiny", False, True), ("prefill", False, True)])
def test_chain_replays_from_a_graph(nrc, name, fused, one_call):
    """Eager chain -> reference kv and caches; the same calls captured into
    a graph on a side stream; three replays, each from reset outputs, each
    equal to the reference bit for bit, with an eager chain on a second
    buffer set and a synchronisation between replays. Covers the split
    projection (tiny, prefill: workspace from the graph's memory pool and a
    second adding kernel), the one-pass projection (weightless), the fused
    form, and the projection + store in one call (its store kernel adding
    the split's partial sums; its eager bits also equal to the three
    calls')."""
    from norm_rope_cache_amd import synth

    cfg = synth.CONFIGS[name]
    d = synth.make_inputs(cfg, with_cache=True)
    _say(f"graph {name} fused={fused} one_call={one_call}: L={cfg.L} T={cfg.T} N={cfg.N}")
    a, b = _Chain(nrc, cfg, d, fused, one_call), _Chain(nrc, cfg, d, fused, one_call)
    a.reset()
    a.run()
    torch.cuda.synchronize()
    ref_kv, ref_caches = to_host(a.kv), to_host(a.caches)
    if one_call:
        three = _Chain(nrc, cfg, d, False)
        three.reset()
        three.run()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(three.kv), ref_kv), "one call: kv differs from the three calls"
        assert np.array_equal(to_host(three.caches), ref_caches), "one call: caches differ from the three calls"
        del three
    assert not np.array_equal(ref_caches, to_host(a.caches0)), "the chain wrote no cache cell"

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        a.reset()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            a.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        a.reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(a.kv), ref_kv), f"replay {rep}: kv differs from the eager chain"
        assert np.array_equal(to_host(a.caches), ref_caches), f"replay {rep}: caches differ from the eager chain"
        b.reset()
        b.run()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(b.caches), ref_caches), f"eager chain after replay {rep} differs"


def test_chains_on_two_explicit_streams(nrc):
    """Two buffer sets run the chain concurrently, each on its own stream
    passed to every call (`stream=`), with the split projection's
    workspace recorded on that stream; each equals the chain run on the
    current stream, bit for bit."""
    from norm_rope_cache_amd import synth

    cfg = synth.CONFIGS["prefill"]
    d = synth.make_inputs(cfg, with_cache=True)
    ref = _Chain(nrc, cfg, d, False)
    ref.reset()
    ref.run()
    torch.cuda.synchronize()
    ref_kv, ref_caches = to_host(ref.kv), to_host(ref.caches)
    del ref

    sets = [_Chain(nrc, cfg, d, False) for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    for c in sets:
        c.reset()
    torch.cuda.synchronize()
    for rep in range(3):
        for c, s in zip(sets, streams):
            s.wait_stream(torch.cuda.current_stream())
            nrc.context_norms(c.x, c.hw, c.pw, cfg.L, d["hidden_eps"], d["pre_eps"], out=c.normed, stream=s)
            nrc.context_kv_project(c.normed, c.w, out=c.kv, stream=s)
            nrc.context_kv_store(c.kv, c.pos, c.slots, c.cs, c.caches, cfg.H, d["k_eps"], stream=s)
        torch.cuda.synchronize()
        for i, c in enumerate(sets):
            assert np.array_equal(to_host(c.kv), ref_kv), f"stream {i}, pass {rep}: kv differs"
            assert np.array_equal(to_host(c.caches), ref_caches), f"stream {i}, pass {rep}: caches differ"
            c.reset()
        torch.cuda.synchronize()
