"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: bit-exact for the norms, the K-norm/RoPE/insert and the scalar
primitives; the projection within 1e-2 relative of the oracle's FP32 sums
(per layer in Frobenius norm and per element against |C*| + the row's RMS).
Inputs come from the seeded generator (norm_rope_cache_amd.synth) and are
handed to both sides; nothing the HIP path computes feeds the oracle.
"""

import numpy as np
import pytest

from helpers import assert_bits_equal, f32, oracle_norms_chunked, projection_tolerance_ok, to_dev, to_host

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


# ------------------------------------------------------------ scalar primitives

def test_scalars_exhaustive(nrc, oracle):
    """The device bf16 rounding and 1/sqrt on all 2^32 f32 patterns equal the
    oracle's (NaN results compared as NaN for 1/sqrt); the paired hardware
    conversion the norms use on NaN-free rows equals it on every non-NaN
    input."""
    from concurrent.futures import ThreadPoolExecutor

    step = 1 << 27
    pool = ThreadPoolExecutor(8)
    for start in range(0, 1 << 32, step):
        _say(f"scalars chunk {start:#x}")
        bits = np.arange(step, dtype=np.uint32) + np.uint32(start)
        x = bits.view(np.float32)
        xd = torch.from_numpy(x).cuda()
        bf, rs = nrc.check_scalars(xd)
        pair = nrc.check_bf16_pair(xd).cpu().numpy().view(np.uint16)
        gb = bf.cpu().numpy().view(np.uint16)
        gr = rs.cpu().numpy()
        parts = np.array_split(np.arange(step), 8)
        ob = np.empty(step, dtype=np.uint16)
        orr = np.empty(step, dtype=np.float32)

        def one(ix):
            ob[ix[0]:ix[-1] + 1] = oracle.bf16(x[ix[0]:ix[-1] + 1])
            orr[ix[0]:ix[-1] + 1] = oracle.rs(x[ix[0]:ix[-1] + 1])

        list(pool.map(one, parts))
        assert_bits_equal(gb, ob, f"bf16 chunk {start:#x}")
        nan = np.isnan(x)
        assert_bits_equal(np.where(nan, 0, pair), np.where(nan, 0, ob), f"paired bf16 chunk {start:#x} (non-NaN)")
        # the fused projection feeds these conversions to the matrix cores,
        # where any NaN operand gives a NaN sum: every NaN must stay a NaN
        pn = pair[nan]
        assert (((pn & 0x7F80) == 0x7F80) & ((pn & 0x7F) != 0)).all(), f"paired bf16 chunk {start:#x}: NaN lost"
        same = (gr.view(np.uint32) == orr.view(np.uint32)) | (np.isnan(gr) & np.isnan(orr))
        if not same.all():
            i = int(np.nonzero(~same)[0][0])
            raise AssertionError(f"rsqrt at {bits[i]:#x}: {gr[i]!r} vs {orr[i]!r}")


# --------------------------------------------------------------------- norms

NORM_CASES = ["tiny", "prefill", "weightless", "long", "edge"]


_INPUTS = {}


def _norms_inputs(name):
    """The workload's inputs without caches, generated once per module (the
    edge workload's take a while); callers must not modify them."""
    from norm_rope_cache_amd import synth

    cfg = synth.CONFIGS[name]
    if name not in _INPUTS:
        _INPUTS[name] = synth.make_inputs(cfg, with_cache=False)
    return cfg, _INPUTS[name]


@pytest.mark.parametrize("name", NORM_CASES)
def test_norms_parity_configs(nrc, oracle, name):
    """Full-size norms, bit-exact over every output element of every config
    (the edge config's 32768 x 8 rows against the oracle in row chunks)."""
    cfg, d = _norms_inputs(name)
    _say(f"norms {name}: L={cfg.L} T={cfg.T}")
    x = to_dev(d["x"])
    hw = None if d["hidden_w"] is None else to_dev(d["hidden_w"])
    pw = None if d["pre_w"] is None else to_dev(d["pre_w"])
    out = nrc.context_norms(x, hw, pw, cfg.L, d["hidden_eps"], d["pre_eps"])
    torch.cuda.synchronize()
    got = to_host(out)
    del out
    if name != "edge":
        want = oracle.context_norms(d["x"], d["hidden_w"], d["pre_w"], cfg.L, d["hidden_eps"], d["pre_eps"])
        assert_bits_equal(got, want, f"norms {name}")
        return

    def cmp(r0, r1, want):
        assert_bits_equal(got[:, r0:r1], want, f"norms edge rows {r0}..{r1 - 1}")

    oracle_norms_chunked(oracle, d["x"], d["hidden_w"], d["pre_w"], cfg.L, d["hidden_eps"], d["pre_eps"],
                         chunk=2048, each=cmp)
    # what the edge rows exercise: about 1% all-zero rows, a few rows with a
    # finite hidden sum, and all others overflowing to signed-zero outputs
    nonzero = np.any((got & 0x7FFF) != 0, axis=(0, 2))
    assert 0 < int(nonzero.sum()) < 64, int(nonzero.sum())


@pytest.mark.parametrize("T", [1, 3, 37, 1000])
@pytest.mark.parametrize("L,hw,pw", [(1, True, True), (2, False, True), (3, True, False), (5, False, False),
                                     (8, True, True), (9, True, True), (12, False, True)])
def test_norms_shapes(nrc, oracle, T, L, hw, pw):
    from norm_rope_cache_amd import synth

    seed = 1000 + 17 * T + L
    x = synth.normal_bf16(seed, (T, 8192), std=1.3)
    w_h = synth.normal_bf16(seed + 1, (8192,), 1.0, 0.1) if hw else None
    w_p = synth.normal_bf16(seed + 2, (L, 8192), 1.0, 0.1) if pw else None
    _say(f"norms T={T} L={L} hw={hw} pw={pw}")
    out = nrc.context_norms(to_dev(x), None if w_h is None else to_dev(w_h), None if w_p is None else to_dev(w_p), L,
                            1e-6, 1e-5)
    want = oracle.context_norms(x, w_h, w_p, L, 1e-6, 1e-5)
    assert_bits_equal(to_host(out), want, f"norms T={T} L={L}")


def test_norms_special_values(nrc, oracle):
    """-0.0, subnormals, near-max values, Inf, NaN, zero rows, -0.0 weights,
    non-zero gain centers and eps = 0."""
    from norm_rope_cache_amd import synth

    T, L = 64, 3
    x = synth.edge_mixture_bf16(77, 78, (T, 8192), nan_inf=True)
    x[5] = 0
    x[6] = 0x8000
    x[7] = synth.edge_mixture_bf16(79, 80, (8192,))  # mixture without NaN/Inf
    x[8, :] = 0x0001  # all smallest subnormals
    x[9, :] = 0x7F7F  # all near max
    x[10] = synth.normal_bf16(81, (8192,))
    x[11] = synth.normal_bf16(82, (8192,), std=1e-20)
    hw = synth.normal_bf16(83, (8192,), 1.0, 0.5)
    hw[::97] = 0x8000
    pw = synth.normal_bf16(84, (L, 8192), 1.0, 0.5)
    pw[:, ::89] = 0x8000
    pw[1, 5] = 0x0003
    for he, pe, hc, pc in [(1e-6, 1e-6, 0.0, 0.0), (0.0, 0.0, 0.0, 0.0), (1e-6, 1e-6, 1.0, -0.5),
                           (1e-6, 1e-6, -0.0, -0.0)]:
        _say(f"norms specials eps={he},{pe} centers={hc},{pc}")
        out = nrc.context_norms(to_dev(x), to_dev(hw), to_dev(pw), L, he, pe, hc, pc)
        want = oracle.context_norms(x, hw, pw, L, he, pe, hc, pc)
        assert_bits_equal(to_host(out), want, f"norms specials {he},{pe},{hc},{pc}")


# ------------------------------------------ norm variants (FP32, input scale)

def _variant_weights(kind, shape, seed):
    from norm_rope_cache_amd import synth

    if kind is None:
        return None
    if kind == "bf16":
        return synth.normal_bf16(seed, shape, 1.0, 0.4)
    return synth.normal_f32(seed, shape, 1.0, 0.4)


@pytest.mark.parametrize("hk", [None, "bf16", "f32"])
@pytest.mark.parametrize("pk", [None, "bf16", "f32"])
def test_norms_ex_parity(nrc, oracle, hk, pk):
    """Every weight kind of each norm, output- and input-scaled, with and
    without gain centers: bit-exact against the oracle on ragged T."""
    from norm_rope_cache_amd import synth

    T, L = 37, 3
    x = synth.normal_bf16(9001, (T, 8192), 0.0, 1.5)
    x[3] = 0
    hw = _variant_weights(hk, (8192,), 9002)
    pw = _variant_weights(pk, (L, 8192), 9003)
    for his in (False, True):
        for pis in (False, True):
            for hc, pc in ((0.0, 0.0), (0.25, -0.5)):
                _say(f"norms_ex hk={hk} pk={pk} in={his},{pis} centers={hc},{pc}")
                got = nrc.context_norms_ex(to_dev(x), None if hw is None else to_dev(hw),
                                           None if pw is None else to_dev(pw), L, 1e-6, 2e-6, hc, pc, his, pis)
                want = oracle.context_norms_ex(x, hw, pw, L, 1e-6, 2e-6, hc, pc, his, pis)
                assert_bits_equal(to_host(got), want, f"norms_ex {hk} {pk} {his} {pis} {hc} {pc}")


def test_norms_ex_special_values_and_grid_stride(nrc, oracle):
    """NaN / Inf / subnormal / near-max rows, -0 and zero FP32 weights, eps = 0,
    and more rows than workgroups (grid stride), both norms input-scaled."""
    from norm_rope_cache_amd import synth

    T, L = 2300, 2
    x = synth.normal_bf16(9101, (T, 8192))
    x[:64] = synth.edge_mixture_bf16(9102, 9103, (64, 8192), nan_inf=True)
    x[64] = 0x8000
    x[65, :] = 0x7F7F
    hw = synth.normal_f32(9104, (8192,), 1.0, 0.5)
    hw[::101] = -0.0
    hw[7] = 0.0
    pw = synth.normal_f32(9105, (L, 8192), 1.0, 0.5)
    pw[1, ::89] = -0.0
    for he, pe, his, pis in ((1e-6, 1e-6, True, True), (0.0, 0.0, True, False), (0.0, 1e-6, False, True)):
        _say(f"norms_ex specials eps={he},{pe} in={his},{pis}")
        got = to_host(nrc.context_norms_ex(to_dev(x), to_dev(hw), to_dev(pw), L, he, pe, 0.0, 0.0, his, pis))
        rows = np.unique(np.concatenate([np.arange(70), np.arange(70, T, 37), [T - 1]]))
        want = oracle.context_norms_ex(np.ascontiguousarray(x[rows]), hw, pw, L, he, pe, 0.0, 0.0, his, pis)
        assert_bits_equal(got[:, rows], want, f"norms_ex specials {he},{pe},{his},{pis}")


@pytest.mark.parametrize("kind,L", [("bf16", 4), ("bf16", 6), ("bf16", 8), ("f32", 4), ("f32", 5)])
def test_norms_ex_layer_counts(nrc, oracle, kind, L):
    """Layer weights staged as FP32 gains (up to 4 layers), as stored bf16 (5
    to 8) and read from memory per row (FP32 beyond 4): bit-exact, both
    scalings, on a row count that is not a multiple of the workgroup's."""
    from norm_rope_cache_amd import synth

    T = 19
    x = synth.normal_bf16(9301, (T, 8192), 0.0, 1.5)
    hw = _variant_weights(kind, (8192,), 9302)
    pw = _variant_weights(kind, (L, 8192), 9303)
    for his, pis in ((False, False), (True, True), (False, True)):
        _say(f"norms_ex layers kind={kind} L={L} in={his},{pis}")
        got = nrc.context_norms_ex(to_dev(x), to_dev(hw), to_dev(pw), L, 1e-6, 2e-6, 0.125, -0.25, his, pis)
        want = oracle.context_norms_ex(x, hw, pw, L, 1e-6, 2e-6, 0.125, -0.25, his, pis)
        assert_bits_equal(to_host(got), want, f"norms_ex layers {kind} {L} {his} {pis}")


def test_norm_gains_overflowing_to_infinity(nrc, oracle):
    """Finite weights whose gain w + center overflows to infinity: zeros of
    the row then give 0 * inf = NaN, which must come out as 0x7FC0 (the
    kernels' hardware conversion is only for rows whose gains are all
    finite). Layer gains overflow under a finite hidden norm; the hidden
    stage is checked on its own output (the fused form's pre-pass)."""
    from norm_rope_cache_amd import synth

    T, L = 9, 2
    x = synth.normal_bf16(9401, (T, 8192), 0.0, 1.0)
    x[:, ::7] = 0
    x[2] = 0
    hw = synth.normal_bf16(9402, (8192,), 1.0, 0.5)
    pw = synth.normal_bf16(9403, (L, 8192), 1.0, 0.5)
    pw[1, ::11] = 0x7F7F  # 3.39e38 + 1e38 = inf in FP32
    for hc in (0.0, 0.5):
        _say(f"norms overflowing layer gains hidden center={hc}")
        got = nrc.context_norms(to_dev(x), to_dev(hw), to_dev(pw), L, 1e-6, 1e-6, hc, 1e38)
        want = oracle.context_norms(x, hw, pw, L, 1e-6, 1e-6, hc, 1e38)
        assert (want == 0x7FC0).any() and ((want & 0x7FFF) == 0x7F80).any()
        assert_bits_equal(to_host(got), want, f"norms overflowing layer gains {hc}")
    hbig = hw.copy()
    hbig[::13] = 0x7F7F
    _say("hidden norm overflowing gains")
    h, _ = nrc.context_hidden_norm(to_dev(x), to_dev(hbig), None, L, 1e-6, 1e-6, 1e38, 0.0)
    want_h, _ = oracle.hidden_norm(x, hbig, 1e-6, 1e38, 1e-6)
    assert (want_h == 0x7FC0).any()
    assert_bits_equal(to_host(h), want_h, "hidden norm overflowing gains")
    hf = synth.normal_f32(9404, (8192,), 1.0, 0.5)
    pf = synth.normal_f32(9405, (L, 8192), 1.0, 0.5)
    pf[0, ::17] = 3e38
    for hwk, pwk in ((hf, pf), (hw, pw), (hf, pw)):
        for his, pis in ((False, False), (True, True), (True, False)):
            _say(f"norms_ex overflowing layer gains {hwk.dtype},{pwk.dtype} in={his},{pis}")
            got = nrc.context_norms_ex(to_dev(x), to_dev(hwk), to_dev(pwk), L, 1e-6, 1e-6, 0.0, 1e38, his, pis)
            want = oracle.context_norms_ex(x, hwk, pwk, L, 1e-6, 1e-6, 0.0, 1e38, his, pis)
            assert_bits_equal(to_host(got), want, f"norms_ex overflowing gains {hwk.dtype} {pwk.dtype} {his} {pis}")


def test_norms_ex_plain_form_is_the_norms(nrc):
    """bf16 weights on the outputs through the general entry: the same bits as
    context_norms (it takes the same kernel)."""
    from norm_rope_cache_amd import synth

    T, L = 300, 4
    x = to_dev(synth.normal_bf16(9201, (T, 8192)))
    hw = to_dev(synth.normal_bf16(9202, (8192,), 1.0, 0.3))
    pw = to_dev(synth.normal_bf16(9203, (L, 8192), 1.0, 0.3))
    a = to_host(nrc.context_norms(x, hw, pw, L, 1e-6, 1e-6, 0.5, 0.0))
    b = to_host(nrc.context_norms_ex(x, hw, pw, L, 1e-6, 1e-6, 0.5, 0.0))
    assert_bits_equal(b, a, "norms_ex plain form")


# ------------------------------------------------------ the residual boundary

def _bw(kind, seed):
    from norm_rope_cache_amd import synth

    if kind is None:
        return None, "bf16"
    w = synth.normal_f32(seed, (8192,), 1.0, 0.4)
    if kind == "bf16":
        return synth.to_bf16_bits(w), "bf16"
    if kind == "f16":
        return w.astype(np.float16).view(np.uint16), "f16"
    return w, "f32"


def _bw_dev(w, kind):
    import torch

    if w is None:
        return None
    if kind == "f16":
        return torch.from_numpy(w.view(np.float16)).cuda()
    return to_dev(w)


@pytest.mark.parametrize("pk", [None, "bf16", "f16", "f32"])
@pytest.mark.parametrize("qk", [None, "bf16", "f16", "f32"])
def test_boundary_parity(nrc, oracle, pk, qk):
    """Every weight kind of each norm, both scalings, FP32 and bf16 streams,
    with and without the stored stream, non-zero centers: the bf16 output and
    the FP32 new stream bit-exact against the oracle."""
    from norm_rope_cache_amd import synth

    m = 37
    x = synth.normal_bf16(9501, (m, 8192), 0.0, 1.5)
    x[4] = 0
    s32 = synth.normal_f32(9502, (m, 8192), 0.0, 2.0)
    alpha = synth.normal_f32(9503, (8192,), 1.0, 0.2)
    beta = synth.normal_f32(9504, (8192,), 0.5, 0.2)
    pw, pks = _bw(pk, 9505)
    qw, qks = _bw(qk, 9506)
    for stream_bf16 in (False, True):
        sin = synth.to_bf16_bits(s32) if stream_bf16 else s32
        for pin, qin in ((False, False), (True, True), (False, True)):
            for store in (True, False):
                _say(f"boundary pk={pk} qk={qk} bf16 stream={stream_bf16} in={pin},{qin} store={store}")
                new_d, out_d = nrc.draft_boundary(to_dev(x), to_dev(sin), to_dev(alpha), to_dev(beta),
                                                  _bw_dev(pw, pks), _bw_dev(qw, qks), 1e-6, 2e-6, 0.125, -0.25,
                                                  pin, qin, store_stream=store)
                new, out = oracle.draft_boundary(x, sin, alpha, beta, pw, qw, 1e-6, 2e-6, 0.125, -0.25, pin, qin,
                                                 pks, qks, store)
                assert_bits_equal(to_host(out_d), out, f"boundary out {pk} {qk} {stream_bf16} {pin} {qin}")
                if store:
                    assert_bits_equal(to_host(new_d).view(np.uint32), new.view(np.uint32),
                                      f"boundary stream {pk} {qk} {stream_bf16} {pin} {qin}")
                else:
                    assert new_d is None


def test_boundary_special_values_and_grid_stride(nrc, oracle):
    """NaN / Inf / subnormal / near-max branch and stream values, zero and
    -0 gates and weights, eps = 0, and more rows than workgroups."""
    from norm_rope_cache_amd import synth

    m = 2300
    x = synth.normal_bf16(9601, (m, 8192))
    x[:64] = synth.edge_mixture_bf16(9602, 9603, (64, 8192), nan_inf=True)
    x[64] = 0x8000
    s = synth.normal_f32(9604, (m, 8192), 0.0, 3.0)
    s[70, ::5] = np.inf
    s[71, ::7] = np.nan
    s[72] = 3e38
    alpha = synth.normal_f32(9605, (8192,), 1.0, 0.2)
    beta = synth.normal_f32(9606, (8192,), 1.0, 0.2)
    alpha[::97] = 0.0
    beta[::89] = -0.0
    pw = synth.normal_f32(9607, (8192,), 1.0, 0.5)
    pw[::101] = -0.0
    qw = synth.to_bf16_bits(synth.normal_f32(9608, (8192,), 1.0, 0.5))
    rows = np.unique(np.concatenate([np.arange(80), np.arange(80, m, 41), [m - 1]]))
    for pe, qe in ((1e-6, 1e-6), (0.0, 0.0)):
        _say(f"boundary specials eps={pe},{qe}")
        new_d, out_d = nrc.draft_boundary(to_dev(x), to_dev(s), to_dev(alpha), to_dev(beta), to_dev(pw), to_dev(qw),
                                          pe, qe)
        new, out = oracle.draft_boundary(np.ascontiguousarray(x[rows]), np.ascontiguousarray(s[rows]), alpha, beta,
                                         pw, qw, pe, qe)
        assert_bits_equal(to_host(out_d)[rows], out, f"boundary specials out {pe}")
        nd = to_host(new_d)[rows]
        same = (nd.view(np.uint32) == new.view(np.uint32)) | (np.isnan(nd) & np.isnan(new))
        assert same.all(), f"boundary specials stream {pe}: {int((~same).sum())} differ"


def test_variants_full_size_as_benchmarked(nrc, oracle):
    """The norm variants and the boundary on the long workload's 16384 rows,
    in the forms bench.py times (FP32 weights with both scalings; FP32 stream
    in and out with bf16 gains): bit-exact on a seeded sample of rows plus the
    first and last (every launch covers all rows; the oracle computes the
    sampled ones)."""
    from norm_rope_cache_amd import synth

    cfg = synth.CONFIGS["long"]
    d = synth.make_inputs(cfg, with_cache=False)
    T, L = cfg.T, cfg.L
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, T - 2, T - 1], rng.choice(T, 160, replace=False)]))
    hw32 = f32(d["hidden_w"])
    pw32 = f32(d["pre_w"])
    x = to_dev(d["x"])
    rows_d = torch.from_numpy(rows).cuda()
    for his in (False, True):
        _say(f"norms_ex full size input-scaled={his}")
        got = to_host(nrc.context_norms_ex(x, to_dev(hw32), to_dev(pw32), L, d["hidden_eps"], d["pre_eps"],
                                           hidden_input_scale=his, pre_input_scale=his)[:, rows_d])
        want = oracle.context_norms_ex(np.ascontiguousarray(d["x"][rows]), hw32, pw32, L, d["hidden_eps"],
                                       d["pre_eps"], 0.0, 0.0, his, his)
        assert_bits_equal(got, want, f"norms_ex full size {his}")
    _say("boundary full size")
    s = synth.normal_f32(9701, (T, 8192), 0.0, 1.0)
    alpha = np.full(8192, 0.9, dtype=np.float32)
    beta = np.full(8192, 1.1, dtype=np.float32)
    new_d, out_d = nrc.draft_boundary(x, to_dev(s), to_dev(alpha), to_dev(beta), to_dev(d["hidden_w"]),
                                      to_dev(np.ascontiguousarray(d["pre_w"][0])))
    new, out = oracle.draft_boundary(np.ascontiguousarray(d["x"][rows]), np.ascontiguousarray(s[rows]), alpha, beta,
                                     d["hidden_w"], np.ascontiguousarray(d["pre_w"][0]))
    assert_bits_equal(to_host(out_d[rows_d]), out, "boundary full size out")
    nd = to_host(new_d[rows_d])
    assert (nd.view(np.uint32) == new.view(np.uint32)).all(), "boundary full size stream"


def test_new_entry_points_edge_cases(nrc, oracle):
    """One row, twelve layers (norm variants), a single boundary row with a
    bf16 stream and FP16 weights, and a store with a non-power-of-two block
    size through strided views: bit-exact against the oracle."""
    import torch
    from norm_rope_cache_amd import synth

    x = synth.normal_bf16(9701, (1, 8192))
    pw = synth.normal_f32(9702, (12, 8192), 1.0, 0.3)
    got = nrc.context_norms_ex(to_dev(x), None, to_dev(pw), 12, 1e-6, 1e-6, 0.0, 0.5, False, True)
    want = oracle.context_norms_ex(x, None, pw, 12, 1e-6, 1e-6, 0.0, 0.5, False, True)
    assert_bits_equal(to_host(got), want, "norms_ex one row, 12 layers")

    s = synth.to_bf16_bits(synth.normal_f32(9703, (1, 8192)))
    a = synth.normal_f32(9704, (8192,), 1.0, 0.1)
    b = synth.normal_f32(9705, (8192,), 1.0, 0.1)
    w16 = synth.normal_f32(9706, (8192,), 1.0, 0.3).astype(np.float16)
    new_d, out_d = nrc.draft_boundary(to_dev(x), to_dev(s), to_dev(a), to_dev(b), torch.from_numpy(w16).cuda(),
                                      torch.from_numpy(w16).cuda(), 1e-5, 1e-5, 0.0, 0.0, True, False)
    new, out = oracle.draft_boundary(x, s, a, b, w16.view(np.uint16), w16.view(np.uint16), 1e-5, 1e-5, 0.0, 0.0,
                                     True, False, "f16", "f16")
    assert_bits_equal(to_host(out_d), out, "boundary one row")
    assert_bits_equal(to_host(new_d).view(np.uint32), new.view(np.uint32), "boundary one row stream")

    L, T, H, bs, nb = 2, 9, 2, 7, 11
    kv = synth.normal_bf16(9707, (L, T, 2 * H * 64))
    pos = np.arange(T, dtype=np.int64)
    tab = synth.to_bf16_bits(np.random.default_rng(5).uniform(-1, 1, (T, 64)))
    slots = [np.random.default_rng(6).permutation(nb * bs)[:T].astype(np.int64), np.array([3, -1, 76], np.int64)]
    bstr, pstr, hstr = H * bs * 136, 136, bs * 136
    size = (nb - 1) * bstr + (bs - 1) * pstr + (H - 1) * hstr + 128
    prior = [synth.random_bits_u16(9710 + l, (size,)) for l in range(L)]
    want = [p.copy() for p in prior]
    oracle.context_kv_store_ex(kv, H, pos, slots, tab, want, bs, nb, bstr, pstr, hstr, 1e-6)
    flats = [to_dev(p) for p in prior]
    views = [torch.as_strided(f, (nb, H, bs, 128), (bstr, hstr, pstr, 1)) for f in flats]
    nrc.context_kv_store_ex(to_dev(kv), to_dev(pos), [to_dev(sl) for sl in slots], to_dev(tab), views, H, 1e-6)
    torch.cuda.synchronize()
    for l in range(L):
        assert_bits_equal(to_host(flats[l]), want[l], f"store_ex block size 7 layer {l}")


# ---------------------------------------------------------------- projection

def _project_check(nrc, oracle, A, B, rows=None, what="", split=True):
    Ad, Bd = to_dev(A), to_dev(B)
    C = to_host(nrc.context_kv_project(Ad, Bd, split=split))
    if rows is not None:
        A_s = np.ascontiguousarray(A[:, rows])
        Cstar = oracle.kv_project(A_s, B)
        C = C[:, rows]
    else:
        Cstar = oracle.kv_project(A, B)
    ok, msg = projection_tolerance_ok(C, Cstar)
    assert ok, f"{what}: {msg}"
    return C


@pytest.mark.parametrize("name", ["tiny", "prefill", "weightless", "long", "edge"])
def test_project_parity_configs(nrc, oracle, name):
    """Full-size projection of every config (the bench's launch shape for
    the long config), checked on sampled rows against the oracle's FP32
    sums."""
    from norm_rope_cache_amd import synth

    cfg = synth.CONFIGS[name]
    _say(f"project {name}: L={cfg.L} T={cfg.T} N={cfg.N}")
    A = synth.bf16_bits_range(cfg.stream(31), (cfg.L, cfg.T, 8192), emin=-4)
    B = synth.normal_bf16(cfg.stream(synth.TID_W), (cfg.L, 8192, cfg.N), std=0.02)
    rng = np.random.default_rng(cfg.index)
    n = min(cfg.T, 24 if cfg.N > 1024 else 64)
    rows = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, n, replace=False)]))
    _project_check(nrc, oracle, A, B, rows, f"project {name}")


@pytest.mark.parametrize("T,N", [(1, 128), (5, 256), (37, 1024), (130, 128), (300, 2048), (513, 384), (1000, 1024)])
@pytest.mark.parametrize("split", [True, False])
def test_project_shapes(nrc, oracle, T, N, split):
    """Ragged T and several N, with the summation split where the shape has
    few tiles (split=True, the default) and in one pass."""
    from norm_rope_cache_amd import synth

    L = 2
    A = synth.normal_bf16(2000 + T, (L, T, 8192))
    B = synth.normal_bf16(3000 + N, (L, 8192, N), std=0.02)
    rows = None if T <= 64 else np.unique(np.concatenate([[0, T - 1], np.arange(1, T, max(1, T // 40))]))
    _say(f"project T={T} N={N} split={split}")
    _project_check(nrc, oracle, A, B, rows, f"project T={T} N={N} split={split}", split=split)


def _expected_k_split(L, T, N, cus=256, nk=256):
    """The split rule written out: none when 256 x 256 tiles fill the CUs;
    else the smallest power of two (each slice an even number of at least 4
    stages of 32) giving one 256 x 256 tile slice per CU (N a multiple of 256,
    at least 256 rows; at most 8 slices) or two 128 x 128 tile slices per CU
    (at most 16 slices)."""
    big_tiles = L * -(-T // 256) * (N // 256)
    if N % 256 == 0 and big_tiles >= cus:
        return 1
    big = N % 256 == 0 and T >= 256
    tiles = big_tiles if big else L * -(-T // 128) * (N // 128)
    target = cus if big else 2 * cus
    s = 1
    while tiles * s < target and s < (8 if big else 16) and nk % (4 * s) == 0 and nk // (2 * s) >= 4:
        s *= 2
    return s


@pytest.mark.parametrize("L,T,N", [(4, 512, 1024), (4, 256, 1024), (1, 130, 128), (2, 300, 384), (2, 16, 256), (4, 2000, 1024),
                                   (1, 700, 512)])
def test_project_split_summation(nrc, oracle, L, T, N):
    """Split summation: the workspace the library asks for follows the split
    rule; the result is within tolerance of the oracle, deterministic, the
    same bits for both weight layouts, and within tolerance of the one-pass
    kernel's."""
    from norm_rope_cache_amd import synth

    lib = nrc._load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = _expected_k_split(L, T, N, cus)
    want_bytes = s * L * T * N * 4 if s > 1 else 0
    assert lib.nrc_context_kv_project_workspace_bytes(L, T, 8192, N) == want_bytes
    A = synth.normal_bf16(4100 + T, (L, T, 8192))
    B = synth.normal_bf16(4200 + N, (L, 8192, N), std=0.02)
    Ad, Bd = to_dev(A), to_dev(B)
    _say(f"project split L={L} T={T} N={N} slices={s}")
    c1 = to_host(nrc.context_kv_project(Ad, Bd))
    c2 = to_host(nrc.context_kv_project(Ad, Bd))
    assert np.array_equal(c1, c2), "split projection not deterministic"
    Bnd = np.ascontiguousarray(np.swapaxes(B, 1, 2))
    c_nd = to_host(nrc.context_kv_project(Ad, to_dev(Bnd), w_layout="nd"))
    assert_bits_equal(c_nd, c1, f"split [L, N, D] vs [L, D, N] {L},{T},{N}")
    c_one = to_host(nrc.context_kv_project(Ad, Bd, split=False))
    rows = np.unique(np.concatenate([[0, T - 1], np.arange(1, T, max(1, T // 40))]))
    Cstar = oracle.kv_project(np.ascontiguousarray(A[:, rows]), B)
    for c, what in ((c1, "split"), (c_one, "one pass")):
        ok, msg = projection_tolerance_ok(c[:, rows], Cstar)
        assert ok, f"{what} L={L} T={T} N={N}: {msg}"



@pytest.mark.parametrize("L,T,N", [(4, 512, 1024), (2, 300, 384), (4, 16384, 1024)])
def test_project_timed_matches_and_stamps(nrc, L, T, N):
    """The clock-stamped projection gives the one-pass kernel's bits, launches
    one workgroup per CU (256 x 256 tiles) or up to two (128 x 128), and every
    workgroup's stamps run forward at a plausible shader clock."""
    from norm_rope_cache_amd import synth

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    A = to_dev(synth.normal_bf16(4300 + T, (L, T, 8192)))
    B = to_dev(synth.normal_bf16(4400 + N, (L, 8192, N), std=0.02))
    _say(f"project timed L={L} T={T} N={N}")
    ref = to_host(nrc.context_kv_project(A, B, split=False))
    out, clk = nrc.context_kv_project_timed(A, B)
    assert_bits_equal(to_host(out), ref, f"timed projection {L},{T},{N}")
    big = N % 256 == 0 and L * ((T + 255) // 256) * (N // 256) >= cus
    tiles = L * ((T + 255) // 256) * (N // 256) if big else L * ((T + 127) // 128) * (N // 128)
    assert clk["workgroups"] == min(tiles, cus if big else 2 * cus)
    st = clk["stamps"]
    assert st.shape == (clk["workgroups"], 4)
    assert bool((st[:, 2] > st[:, 0]).all()) and bool((st[:, 3] > st[:, 1]).all())
    assert clk["wall_khz"] > 0
    ghz = clk["shader_ghz"]
    assert float(ghz.min()) > 0.05 and float(ghz.max()) < 5.0, (float(ghz.min()), float(ghz.max()))
    _say(f"  shader clock GHz median {float(ghz.median()):.3f}")
    z, clk0 = nrc.context_kv_project_timed(A[:, :0], B)
    assert clk0["workgroups"] == 0 and z.shape == (L, 0, N)


@pytest.mark.parametrize("D", [192, 320, 640, 1088])
@pytest.mark.parametrize("T", [40, 1300])
def test_project_other_summation_lengths(nrc, oracle, D, T):
    """Summation lengths other than 8192 (any multiple of 64): the one-pass
    and split forms (few rows split D when the split rule allows an even
    number of 32-wide stages per slice) and both weight layouts, within
    tolerance of the oracle; the two layouts give the same bits."""
    from norm_rope_cache_amd import synth

    L, N = 2, 256
    A = synth.normal_bf16(4500 + D, (L, T, D))
    B = synth.normal_bf16(4600 + D, (L, D, N), std=0.02)
    Ad, Bd = to_dev(A), to_dev(B)
    _say(f"project D={D} T={T}")
    Cstar = oracle.kv_project(A, B)
    outs = {}
    for split in (False, True):
        c = to_host(nrc.context_kv_project(Ad, Bd, split=split))
        ok, msg = projection_tolerance_ok(c, Cstar)
        assert ok, f"D={D} T={T} split={split}: {msg}"
        outs[split] = c
    c_nd = to_host(nrc.context_kv_project(Ad, to_dev(np.ascontiguousarray(np.swapaxes(B, 1, 2))), w_layout="nd"))
    assert_bits_equal(c_nd, outs[True], f"[L, N, D] vs [L, D, N] D={D} T={T}")

@pytest.mark.parametrize("L,T,N", [(4, 3000, 1024), (2, 4196, 2048), (1, 8292, 2560)])
def test_project_several_tiles_per_workgroup(nrc, oracle, L, T, N):
    """Shapes with more output tiles than resident workgroups, so each
    workgroup walks several tiles: 768 tiles of 128 x 128 (ragged last row
    tile), 272 tiles of 256 x 256 (split evenly over the XCDs) and 330 of
    256 x 256 (not a multiple of 8: round-robin assignment). Sampled rows,
    the ragged tail included, against the oracle's FP32 sums."""
    from norm_rope_cache_amd import synth

    A = synth.normal_bf16(5000 + T, (L, T, 8192))
    B = synth.normal_bf16(6000 + N, (L, 8192, N), std=0.02)
    rows = np.unique(np.concatenate([[0, T - 1], np.arange(1, T, max(1, T // 48)), np.arange(T - 60, T)]))
    _say(f"project multi-tile L={L} T={T} N={N}")
    _project_check(nrc, oracle, A, B, rows, f"project multi-tile L={L} T={T} N={N}")


@pytest.mark.parametrize("L,T,N,split", [(5, 2000, 2048, False), (5, 300, 2048, False), (5, 300, 2048, True)])
def test_project_weights_beyond_half_the_infinity_cache(nrc, oracle, L, T, N, split):
    """Stacked weights over 128 MB take the layer-synchronous tile order:
    320 tiles of 256 x 256 over 256 workgroups (a ragged last round on two
    XCDs and a ragged last row tile), 128 x 128 tiles in one pass, and the
    split form; sampled rows against the oracle."""
    from norm_rope_cache_amd import synth

    assert L * 8192 * N * 2 > (128 << 20)
    A = synth.normal_bf16(8100 + T, (L, T, 8192))
    B = synth.normal_bf16(8200 + N, (L, 8192, N), std=0.02)
    rows = np.unique(np.concatenate([[0, T - 1], np.arange(1, T, max(1, T // 24))]))
    _say(f"project large weights L={L} T={T} N={N} split={split}")
    _project_check(nrc, oracle, A, B, rows, f"project large weights {L},{T},{N}", split=split)


@pytest.mark.parametrize("L,T,N", [(2, 37, 256), (4, 300, 1024), (1, 513, 384), (4, 16384, 1024)])
def test_project_nd_weight_layout(nrc, oracle, L, T, N):
    """The pages' [L, N, D] weight storage: the same bits as the [L, D, N]
    layout (same sums in the same order), and within tolerance of the
    oracle's [L, N, D] routine on sampled rows (the last shape is the long
    workload's launch)."""
    from norm_rope_cache_amd import synth

    A = synth.normal_bf16(8100 + T, (L, T, 8192))
    Bnd = synth.normal_bf16(8200 + N, (L, N, 8192), std=0.02)
    Bdn = np.ascontiguousarray(Bnd.transpose(0, 2, 1))
    _say(f"project nd L={L} T={T} N={N}")
    Ad = to_dev(A)
    c_nd = to_host(nrc.context_kv_project(Ad, to_dev(Bnd), w_layout="nd"))
    c_dn = to_host(nrc.context_kv_project(Ad, to_dev(Bdn)))
    assert_bits_equal(c_nd, c_dn, f"nd vs dn L={L} T={T} N={N}")
    rows = np.unique(np.concatenate([[0, T - 1], np.arange(1, T, max(1, T // 24))]))
    Cstar = oracle.kv_project_nd(np.ascontiguousarray(A[:, rows]), Bnd)
    ok, msg = projection_tolerance_ok(c_nd[:, rows], Cstar)
    assert ok, msg


def test_project_one_hot_and_zero_rows(nrc, oracle):
    """A one-hot row selects a row of B: the result is that row's bf16 value
    exactly; an all-zero row gives +0."""
    from norm_rope_cache_amd import synth

    L, T, N = 2, 300, 1024
    B = synth.normal_bf16(4001, (L, 8192, N), std=0.02)
    A = np.zeros((L, T, 8192), dtype=np.uint16)
    cols = (np.arange(T) * 97) % 8192
    for l in range(L):
        A[l, np.arange(T - 10), cols[:T - 10]] = 0x3F80
    C = to_host(nrc.context_kv_project(to_dev(A), to_dev(B)))
    for l in range(L):
        assert_bits_equal(C[l, :T - 10], B[l, cols[:T - 10]], f"one-hot rows layer {l}")
        assert np.all(C[l, T - 10:] == 0)


# -------------------------------------------------- store: full operand surface

@pytest.mark.parametrize("layout", ["head-major padded", "page-major", "backend contiguous"])
def test_store_ex_strided_views_and_slot_groups(nrc, oracle, layout):
    """Per-layer slot lists of their own lengths, None layers (no store),
    more than 8 layers (two launches) and strided cache views: every element
    of each layer's flat buffer (padding included) equals the oracle's."""
    import torch
    from norm_rope_cache_amd import synth

    L, T, H, bs, nb = 10, 40, 4, 8, 24
    N = 2 * H * 64
    rng = np.random.default_rng(33)
    kv = synth.normal_bf16(3301, (L, T, N), 0.0, 1.5)
    pos = rng.integers(0, 128, T).astype(np.int64)
    tab = synth.to_bf16_bits(rng.uniform(-1, 1, (128, 64)))
    lens = [40, 0, 17, None, 40, 5, None, 33, 40, 1]
    slots = []
    for l, n in enumerate(lens):
        if n is None:
            slots.append(None)
            continue
        sl = rng.permutation(nb * bs)[:n].astype(np.int64)
        sl[rng.random(n) < 0.2] = -1
        slots.append(sl)
    bstr, pstr, hstr = {"head-major padded": (H * bs * 136 + 64, 136, bs * 136),
                        "page-major": (bs * H * 128, H * 128, 128),
                        "backend contiguous": (H * bs * 128, 128, bs * 128)}[layout]
    size = (nb - 1) * bstr + (bs - 1) * pstr + (H - 1) * hstr + 128
    prior = [synth.random_bits_u16(3400 + l, (size,)) for l in range(L)]
    want = [p.copy() for p in prior]
    oracle.context_kv_store_ex(kv, H, pos, slots, tab, want, bs, nb, bstr, pstr, hstr, 1e-6)
    flats = [to_dev(p) for p in prior]
    views = [torch.as_strided(f, (nb, H, bs, 128), (bstr, hstr, pstr, 1)) for f in flats]
    _say(f"store_ex {layout}")
    nrc.context_kv_store_ex(to_dev(kv), to_dev(pos), [None if sl is None else to_dev(sl) for sl in slots],
                            to_dev(tab), [v if sl is not None else None for v, sl in zip(views, slots)], H, 1e-6)
    torch.cuda.synchronize()
    for l in range(L):
        assert_bits_equal(to_host(flats[l]), want[l], f"store_ex {layout} layer {l}")


def test_store_ex_matches_store_on_contiguous_caches(nrc):
    """The general entry on contiguous caches with one slot length is the
    plain store (same kernel, same bits)."""
    import torch
    from norm_rope_cache_amd import synth

    cfg = synth.scaled(synth.PREFILL, 300)
    d = synth.make_inputs(cfg, with_cache=True, kv_synth=True, with_x=False, with_weights=False)
    a = to_dev(d["caches"])
    b = to_dev(d["caches"])
    kv, pos, cs = to_dev(d["kv"]), to_dev(d["positions"]), to_dev(d["cos_sin"])
    slots = to_dev(d["slots"])
    nrc.context_kv_store(kv, pos, slots, cs, a, cfg.H, d["k_eps"])
    nrc.context_kv_store_ex(kv, pos, [slots[l] for l in range(cfg.L)], cs, [b[l] for l in range(cfg.L)], cfg.H,
                            d["k_eps"])
    torch.cuda.synchronize()
    assert_bits_equal(to_host(b), to_host(a), "store_ex vs store")


# -------------------------------------------------------------------- store

def _store_case(name, T=None, kv_rows=4096):
    from norm_rope_cache_amd import synth

    cfg = synth.CONFIGS[name]
    if T is not None:
        cfg = synth.scaled(cfg, T)
    d = synth.make_inputs(cfg, with_cache=True, kv_synth=cfg.T <= kv_rows, with_x=False, with_weights=False)
    if "kv" not in d:
        # a block of synthetic projection rows repeated over T (bounded generation)
        if cfg.edge:
            blk = synth.edge_mixture_bf16(cfg.stream(synth.TID_KVMIX), cfg.stream(synth.TID_KV),
                                          (cfg.L, kv_rows, cfg.N), nan_inf=True)
        else:
            blk = synth.normal_bf16(cfg.stream(synth.TID_KV), (cfg.L, kv_rows, cfg.N), std=1.8)
        reps = (cfg.T + kv_rows - 1) // kv_rows
        d["kv"] = np.ascontiguousarray(np.tile(blk, (1, reps, 1))[:, :cfg.T])
    return cfg, d


def _run_store(nrc, oracle, cfg, d, rows=None, eps=1e-6):
    caches_d = to_dev(d["caches"])
    kv_d = to_dev(d["kv"])
    slots = d["slots"] if rows is None else np.ascontiguousarray(d["slots"][:, :rows])
    slots_d = to_dev(slots)
    cs_d = None if d["cos_sin"] is None else to_dev(d["cos_sin"])
    pos_d = to_dev(d["positions"])
    nrc.context_kv_store(kv_d, pos_d, slots_d, cs_d, caches_d, cfg.H, eps)
    torch.cuda.synchronize()
    got = to_host(caches_d)
    want = d["caches"].copy()
    oracle.context_kv_store(d["kv"], cfg.H, d["positions"], slots, d["cos_sin"], want, cfg.block_size, eps)
    return got, want


@pytest.mark.parametrize("name", ["tiny", "prefill", "weightless", "long", "edge"])
def test_store_parity_configs(nrc, oracle, name):
    """Full-size K-norm + RoPE + insert, bit-exact over every cache cell
    (untouched cells keep their prior random bits)."""
    cfg, d = _store_case(name)
    _say(f"store {name}: L={cfg.L} T={cfg.T} H={cfg.H} bs={cfg.block_size} nb={cfg.num_blocks}")
    got, want = _run_store(nrc, oracle, cfg, d)
    assert_bits_equal(got, want, f"store {name}")


def test_store_from_oracle_projection(nrc, oracle):
    """The store on a realistic projection output: the oracle's chain up to
    the projection (norms, FP32 sums, bf16) feeds both sides."""
    from norm_rope_cache_amd import synth

    cfg = synth.scaled(synth.PREFILL, 64)
    d = synth.make_inputs(cfg, with_cache=True)
    normed = oracle.context_norms(d["x"], d["hidden_w"], d["pre_w"], cfg.L)
    d["kv"] = oracle.bf16(oracle.kv_project(normed, d["w_kv"]))
    got, want = _run_store(nrc, oracle, cfg, d)
    assert_bits_equal(got, want, "store on the oracle's projection")


def test_store_rows_subset_and_rope_off(nrc, oracle):
    """Only the first `rows` rows are inserted; RoPE off stores the K-norm."""
    cfg, d = _store_case("tiny")
    for rows in (0, 1, 7, 16):
        _say(f"store tiny rows={rows}")
        got, want = _run_store(nrc, oracle, cfg, d, rows=rows)
        assert_bits_equal(got, want, f"store rows={rows}")
    d["cos_sin"] = None
    got, want = _run_store(nrc, oracle, cfg, d)
    assert_bits_equal(got, want, "store rope off")


@pytest.mark.parametrize("L,H,bs,nb", [(10, 2, 24, 9), (3, 4, 7, 50), (9, 1, 1, 300), (2, 32, 5, 60)])
def test_store_shapes(nrc, oracle, L, H, bs, nb):
    """More than 8 layers (two launches), block sizes that are not powers of
    two, 1..32 heads, per-layer slot mappings."""
    from norm_rope_cache_amd import synth

    T = 200
    N = 2 * H * 64
    rng = np.random.default_rng(L * 1000 + H)
    kv = synth.normal_bf16(5000 + L + H, (L, T, N), std=1.8)
    slots = np.stack([rng.permutation(nb * bs)[:T] for _ in range(L)]).astype(np.int64)
    slots[rng.random((L, T)) < 0.2] = -1
    positions = rng.integers(0, 512, T).astype(np.int64)
    tab = synth.rope_table(512)
    caches = synth.random_bits_u16(6000 + L, (L, nb, H, bs, 128))
    for eps in (1e-6, 0.0, 0.25):
        _say(f"store shapes L={L} H={H} bs={bs} nb={nb} eps={eps}")
        cd = to_dev(caches)
        nrc.context_kv_store(to_dev(kv), to_dev(positions), [to_dev(s) for s in slots], to_dev(tab),
                             [cd[i] for i in range(L)], H, eps)
        want = caches.copy()
        oracle.context_kv_store(kv, H, positions, slots, tab, want, bs, eps)
        assert_bits_equal(to_host(cd), want, f"store L={L} H={H} bs={bs} eps={eps}")


def test_store_operand_forms(nrc, oracle):
    """The store call's operand forms give the same cache: stacked caches and
    slot rows (addressed by their layer stride), lists of per-layer tensors,
    and stacked tensors with padded layer strides (taken layer by layer)."""
    import torch
    from norm_rope_cache_amd import synth

    L, T, H, bs, nb = 3, 40, 8, 16, 8
    kv = synth.normal_bf16(7101, (L, T, 2 * H * 64), std=1.3)
    rng = np.random.default_rng(71)
    slots = np.stack([rng.permutation(nb * bs)[:T] for _ in range(L)]).astype(np.int64)
    slots[1, 5] = -1
    positions = rng.integers(0, 64, T).astype(np.int64)
    tab = synth.rope_table(64)
    caches = synth.random_bits_u16(7102, (L, nb, H, bs, 128))
    want = caches.copy()
    oracle.context_kv_store(kv, H, positions, slots, tab, want, bs, 1e-6)
    kv_d, pos_d, tab_d = to_dev(kv), to_dev(positions), to_dev(tab)
    _say("store operand forms")
    stacked, slots_d = to_dev(caches), to_dev(slots)
    nrc.context_kv_store(kv_d, pos_d, slots_d, tab_d, stacked, H, 1e-6)
    assert_bits_equal(to_host(stacked), want, "store, stacked caches and slots")
    listed = [to_dev(caches[l]) for l in range(L)]
    nrc.context_kv_store(kv_d, pos_d, [to_dev(slots[l]) for l in range(L)], tab_d, listed, H, 1e-6)
    for l in range(L):
        assert_bits_equal(to_host(listed[l]), want[l], f"store, listed caches, layer {l}")
    padded_c = torch.zeros((L, nb + 1, H, bs, 128), dtype=torch.bfloat16, device="cuda")
    padded_c[:, :nb] = to_dev(caches)
    padded_s = torch.full((L, T + 3), -1, dtype=torch.int64, device="cuda")
    padded_s[:, :T] = slots_d
    nrc.context_kv_store(kv_d, pos_d, padded_s[:, :T], tab_d, padded_c[:, :nb], H, 1e-6)
    got = to_host(padded_c)
    assert_bits_equal(got[:, :nb], want, "store, padded layer strides")
    assert np.all(got[:, nb:] == 0), "store wrote past a layer's cache"


def test_store_strided_views(nrc, oracle):
    """k and v as views with padded row and layer strides."""
    from norm_rope_cache_amd import synth

    L, T, H, bs, nb = 3, 50, 2, 16, 8
    N = 2 * H * 64
    kv = synth.normal_bf16(7001, (L, T, N), std=1.8)
    big = np.zeros((L + 1, T + 3, N + 64), dtype=np.uint16)
    big[:L, :T, :N] = kv
    bd = to_dev(big)
    k = bd[:L, :T, :H * 64].unflatten(2, (H, 64))
    v = bd[:L, :T, H * 64:N].unflatten(2, (H, 64))
    rng = np.random.default_rng(3)
    slots = np.stack([rng.permutation(nb * bs)[:T] for _ in range(L)]).astype(np.int64)
    positions = np.arange(T, dtype=np.int64)
    tab = synth.rope_table(64)
    caches = synth.random_bits_u16(7002, (L, nb, H, bs, 128))
    cd = to_dev(caches)
    nrc.context_kv_store(None, to_dev(positions), to_dev(slots), to_dev(tab), cd, H, 1e-6, k=k, v=v)
    want = caches.copy()
    oracle.context_kv_store(kv, H, positions, slots, tab, want, bs, 1e-6)
    assert_bits_equal(to_host(cd), want, "store strided views")


def test_store_skips_out_of_range_rows(nrc, oracle):
    """Rows whose slot or position breaks the range preconditions are skipped
    by the kernel's own bounds checks (nothing is written out of bounds)."""
    from norm_rope_cache_amd import synth

    L, T, H, bs, nb = 2, 40, 2, 16, 4
    kv = synth.normal_bf16(8001, (L, T, 256), std=1.8)
    rng = np.random.default_rng(5)
    slots = np.stack([rng.permutation(nb * bs)[:T] for _ in range(L)]).astype(np.int64)
    positions = rng.integers(0, 100, T).astype(np.int64)
    tab = synth.rope_table(100)
    bad_slot = slots.copy()
    bad_slot[0, 3] = nb * bs + 5
    bad_slot[1, 4] = 1 << 40
    bad_pos = positions.copy()
    bad_pos[7] = 100
    bad_pos[8] = -3
    caches = synth.random_bits_u16(8002, (L, nb, H, bs, 128))
    cd = to_dev(caches)
    nrc.context_kv_store(to_dev(kv), to_dev(bad_pos), to_dev(bad_slot), to_dev(tab), cd, H, 1e-6)
    # expected: the oracle on the valid rows only (skipped rows as slot -1)
    ok_slots = bad_slot.copy()
    ok_slots[0, 3] = -1
    ok_slots[1, 4] = -1
    ok_slots[:, 7] = -1
    ok_slots[:, 8] = -1
    ok_pos = positions.copy()
    want = caches.copy()
    oracle.context_kv_store(kv, H, ok_pos, ok_slots, tab, want, bs, 1e-6)
    assert_bits_equal(to_host(cd), want, "store with out-of-range rows")



@pytest.mark.parametrize("H", [8, 2])
@pytest.mark.parametrize("eps", [0.0, 1e-6])
def test_store_non_finite_norm_and_rope(nrc, oracle, H, eps):
    """Heads whose K-norm or RoPE meets zero, overflow, Inf and NaN: an
    all-zero head (with eps = 0 its scale is infinite and 0 * inf = NaN), a
    head whose sum of squares overflows (scale 0), heads holding one Inf or
    one NaN, a head of subnormals, and cos/sin rows holding Inf and NaN. Both
    grid forms (H >= 8: one row per wave; H < 8: per-lane rows)."""
    from norm_rope_cache_amd import synth

    L, T, bs, nb = 2, 48, 16, 8
    N = 2 * H * 64
    kv = synth.normal_bf16(8101 + H, (L, T, N), std=1.8)
    kv[:, 1, 0:64] = 0                       # zero K head
    kv[:, 2, 0:64] = 0x7F70                  # sum of squares overflows
    kv[:, 3, 64 * (H - 1) + 5] = 0x7F80      # one +Inf in the last K head
    kv[:, 4, 7] = 0xFFC1                     # one NaN
    kv[:, 5, 0:64] = 0x0003                  # subnormals
    kv[:, 6, 0:64] = 0x8000                  # -0 head
    rng = np.random.default_rng(11)
    slots = np.stack([rng.permutation(nb * bs)[:T] for _ in range(L)]).astype(np.int64)
    positions = np.arange(T, dtype=np.int64) % 20
    tab = synth.rope_table(20)
    tab[9, 3] = 0x7F80                       # cos = +Inf
    tab[10, 32 + 5] = 0x7FC3                 # sin = NaN
    tab[11, :] = 0                           # cos = sin = 0
    positions[12] = 9
    positions[13] = 10
    positions[14] = 11
    positions[1] = 9                         # the zero head meets the Inf cos
    caches = synth.random_bits_u16(8103, (L, nb, H, bs, 128))
    _say(f"store non-finite H={H} eps={eps}")
    cd = to_dev(caches)
    nrc.context_kv_store(to_dev(kv), to_dev(positions), to_dev(slots), to_dev(tab), cd, H, eps)
    want = caches.copy()
    oracle.context_kv_store(kv, H, positions, slots, tab, want, bs, eps)
    assert_bits_equal(to_host(cd), want, f"store non-finite H={H} eps={eps}")


def test_store_ex_heads_beyond_32bit_offsets(nrc, oracle):
    """A cache view whose heads lie more than 2 GiB apart from the first
    (H = 8, one row per wave): the row form cannot address them from one
    32-bit offset and takes the 64-bit address form. The device buffer spans
    2.2 GB; the oracle writes a compact twin with the same block and page
    strides, and each head's region plus a margin after it is compared."""
    import torch
    from norm_rope_cache_amd import synth

    L, T, H, bs, nb = 1, 30, 8, 4, 9
    bstr, pstr = bs * 136, 136
    hs_big = 160_000_000                      # (H - 1) * hs_big * 2 bytes > 2^31
    reg = (nb - 1) * bstr + (bs - 1) * pstr + 128 + 1024
    hs_c = (reg + 7) // 8 * 8
    rng = np.random.default_rng(77)
    kv = synth.normal_bf16(7701, (L, T, 2 * H * 64), std=1.4)
    pos = rng.integers(0, 64, T).astype(np.int64)
    tab = synth.to_bf16_bits(rng.uniform(-1, 1, (64, 64)))
    slots = [rng.permutation(nb * bs)[:T].astype(np.int64)]
    compact = synth.random_bits_u16(7702, ((H - 1) * hs_c + reg,))
    want = compact.copy()
    oracle.context_kv_store_ex(kv, H, pos, slots, tab, [want], bs, nb, bstr, pstr, hs_c, 1e-6)
    _say("store_ex heads 2.2 GB apart")
    flat = torch.empty(((H - 1) * hs_big + reg,), dtype=torch.bfloat16, device="cuda")
    for h in range(H):
        flat[h * hs_big:h * hs_big + reg] = to_dev(compact[h * hs_c:h * hs_c + reg])
    view = torch.as_strided(flat, (nb, H, bs, 128), (bstr, hs_big, pstr, 1))
    nrc.context_kv_store_ex(to_dev(kv), to_dev(pos), [to_dev(s) for s in slots], to_dev(tab), [view], H, 1e-6)
    torch.cuda.synchronize()
    for h in range(H):
        assert_bits_equal(to_host(flat[h * hs_big:h * hs_big + reg]), want[h * hs_c:h * hs_c + reg],
                          f"store_ex far heads, head {h}")
    del flat, view
    torch.cuda.empty_cache()

# --------------------------------------------------------------------- chain

@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name,T", [("tiny", 16), ("prefill", 48), ("weightless", 40)])
def test_chain_parity(nrc, oracle, name, T, fused):
    """The chain through all three calls against the oracle's chain: norms
    bit-exact, projection within tolerance, cache cells written exactly where
    the oracle writes them, with K and V within the projection's tolerance
    and every other cell untouched."""
    from norm_rope_cache_amd import synth

    cfg = synth.scaled(synth.CONFIGS[name], T)
    d = synth.make_inputs(cfg, with_cache=True)
    _say(f"chain {name} T={T} fused={fused}")
    caches_d = to_dev(d["caches"])
    L = cfg.L
    normed = torch.empty((L, cfg.T, 8192), dtype=torch.bfloat16, device="cuda")
    kv = nrc.context_kv_chain(
        to_dev(d["x"]), None if d["hidden_w"] is None else to_dev(d["hidden_w"]),
        None if d["pre_w"] is None else to_dev(d["pre_w"]), to_dev(d["w_kv"]), to_dev(d["positions"]),
        to_dev(d["slots"]), None if d["cos_sin"] is None else to_dev(d["cos_sin"]), caches_d, cfg.H,
        fused=fused, workspace=None if fused else normed)
    torch.cuda.synchronize()
    want_caches = d["caches"].copy()
    o_normed, o_kv = oracle.chain(d["x"], d["hidden_w"], d["pre_w"], cfg.L, d["w_kv"], cfg.H, d["positions"],
                                  d["slots"], d["cos_sin"], want_caches, cfg.block_size)
    if not fused:
        assert_bits_equal(to_host(normed), o_normed, f"chain norms {name}")
    ok, msg = projection_tolerance_ok(to_host(kv), oracle.kv_project(o_normed, d["w_kv"]))
    assert ok, msg
    got_caches = to_host(caches_d)
    written = np.any(want_caches != d["caches"], axis=-1) | np.any(got_caches != d["caches"], axis=-1)
    assert_bits_equal(got_caches[~written], d["caches"][~written], "untouched cells")
    # every written cell: K within tolerance of the oracle's K, V likewise
    gw = f32(got_caches[written]).astype(np.float64)
    ww = f32(want_caches[written]).astype(np.float64)
    err = np.abs(gw - ww)
    assert np.all(err <= 2e-2 * (np.abs(ww) + np.sqrt(np.mean(ww ** 2, axis=-1, keepdims=True)))), \
        f"chain cache values: max error {err.max()}"


def _finite_edge_rows(d):
    """Rows of the edge workload whose hidden sum of squares stays finite (no
    value near the bf16 maximum) and that are not all zero: the only rows
    whose norms, and so projections, are not all signed zeros."""
    x = d["x"]
    big = ((x & 0x7FFF) >= 0x7F70).any(axis=1)
    zero = ~((x & 0x7FFF) != 0).any(axis=1)
    return np.nonzero(~big & ~zero)[0]


CHAIN_FULL = [(n, False) for n in NORM_CASES] + [("long", True)]


@pytest.mark.parametrize("name,fused", CHAIN_FULL)
def test_chain_full_size_store_bitwise(nrc, oracle, name, fused):
    """The whole chain at full size in the launch configuration bench.py
    times (one slot mapping shared by every layer; the projection split for
    small T). Every cache cell equals the oracle's store run on the GPU's own
    projection output, bit for bit (the pages' store reads the bmm's own
    output), untouched cells included. The projection is checked within its
    tolerance on sampled rows against the oracle's FP32 sums of the oracle's
    norms (edge: every row whose norms are not all zero, fed with those rows'
    real norms; every other row must project to signed zeros)."""
    from norm_rope_cache_amd import synth

    cfg, d = _norms_inputs(name)
    _say(f"chain full size {name} fused={fused}: L={cfg.L} T={cfg.T} N={cfg.N}")
    caches = synth.random_bits_u16(cfg.stream(synth.TID_CACHE), (cfg.L, cfg.num_blocks, cfg.H, cfg.block_size, 128))
    caches_d = to_dev(caches)
    x_d = to_dev(d["x"])
    hw = None if d["hidden_w"] is None else to_dev(d["hidden_w"])
    pw = None if d["pre_w"] is None else to_dev(d["pre_w"])
    w_d = to_dev(d["w_kv"])
    pos_d = to_dev(d["positions"])
    slots_d = to_dev(d["slots"][0])  # one mapping, every layer
    cs_d = None if d["cos_sin"] is None else to_dev(d["cos_sin"])
    normed = None
    if fused:
        h, r = nrc.context_hidden_norm(x_d, hw, pw, cfg.L, d["hidden_eps"], d["pre_eps"])
        kv = nrc.context_kv_project_fused(h, r, pw, w_d)
        del h, r
    else:
        normed = nrc.context_norms(x_d, hw, pw, cfg.L, d["hidden_eps"], d["pre_eps"])
        kv = nrc.context_kv_project(normed, w_d)
    nrc.context_kv_store(kv, pos_d, slots_d, cs_d, caches_d, cfg.H, d["k_eps"])
    torch.cuda.synchronize()
    kv_h = to_host(kv)
    got = to_host(caches_d)
    del caches_d, kv
    oracle.context_kv_store(kv_h, cfg.H, d["positions"], d["slots"], d["cos_sin"], caches, cfg.block_size,
                            d["k_eps"])
    assert_bits_equal(got, caches, f"chain {name}: cache vs the oracle's store of the GPU projection")
    del got, caches

    rng = np.random.default_rng(cfg.index + 11)
    if cfg.edge:
        rows = _finite_edge_rows(d)
        assert rows.size > 0
        others = np.ones(cfg.T, dtype=bool)
        others[rows] = False
        assert not np.any((kv_h[:, others] & 0x7FFF) != 0), "edge: a row with all-zero norms projected to non-zero"
    else:
        n = min(cfg.T, 40)
        rows = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, n, replace=False)]))
    on = oracle.context_norms(np.ascontiguousarray(d["x"][rows]), d["hidden_w"], d["pre_w"], cfg.L,
                              d["hidden_eps"], d["pre_eps"])
    if normed is not None:
        assert_bits_equal(to_host(normed[:, torch.from_numpy(rows).cuda()]), on, f"chain {name}: norms")
    ok, msg = projection_tolerance_ok(kv_h[:, rows], oracle.kv_project(on, d["w_kv"]))
    assert ok, f"chain {name}: projection: {msg}"


@pytest.mark.parametrize("fused", [False, True])
def test_deterministic(nrc, fused):
    """Two runs of the chain give identical bits."""
    from norm_rope_cache_amd import synth

    cfg = synth.scaled(synth.PREFILL, 300)
    d = synth.make_inputs(cfg, with_cache=True)
    outs = []
    for _ in range(2):
        cd = to_dev(d["caches"])
        kv = nrc.context_kv_chain(to_dev(d["x"]), to_dev(d["hidden_w"]), to_dev(d["pre_w"]), to_dev(d["w_kv"]),
                                  to_dev(d["positions"]), to_dev(d["slots"]), to_dev(d["cos_sin"]), cd, cfg.H,
                                  fused=fused, split=False)
        outs.append((to_host(kv), to_host(cd)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


# --------------------------------------------------- fused norms + projection

@pytest.mark.parametrize("name", ["tiny", "prefill", "weightless", "long", "edge"])
def test_hidden_norm_parity_configs(nrc, oracle, name):
    """Pre-pass of the fused path: h bit-exact and |r| bit-exact against the
    oracle's hidden norm and layer-norm scale (edge: sampled rows incl. every
    zero row and every finite-sum row)."""
    cfg, d = _norms_inputs(name)
    _say(f"hidden norm {name}: T={cfg.T}")
    h, r = nrc.context_hidden_norm(to_dev(d["x"]), None if d["hidden_w"] is None else to_dev(d["hidden_w"]),
                                   None if d["pre_w"] is None else to_dev(d["pre_w"]), cfg.L, d["hidden_eps"],
                                   d["pre_eps"])
    torch.cuda.synchronize()
    if name == "edge":
        xf = f32(d["x"])
        finite_rows = np.nonzero(np.isfinite((xf.astype(np.float64) ** 2).sum(axis=1)))[0]
        rng = np.random.default_rng(98)
        rows = np.unique(np.concatenate([d["zero_rows"], finite_rows, rng.choice(cfg.T, 512, replace=False)]))
    else:
        rows = np.arange(cfg.T)
    oh, orr = oracle.hidden_norm(np.ascontiguousarray(d["x"][rows]), d["hidden_w"], d["hidden_eps"], 0.0,
                                 d["pre_eps"])
    ridx = torch.from_numpy(rows).cuda()
    assert_bits_equal(to_host(h[ridx]), oh, f"hidden norm h {name}")
    gr = np.abs(r[ridx].cpu().numpy())
    same = (gr.view(np.uint32) == np.abs(orr).view(np.uint32)) | (np.isnan(gr) & np.isnan(orr))
    assert same.all(), f"hidden norm r {name}: {np.nonzero(~same)[0][:5]}"


def _fused_vs_unfused(nrc, x, hw, pw, w_kv, L, he=1e-6, pe=1e-6, hc=0.0, pc=0.0, split=False):
    """(unfused kv, fused kv), both in one pass (split=False) or both with
    the summation split where the shape splits (split=True)."""
    xd, wd = to_dev(x), to_dev(w_kv)
    hwd = None if hw is None else to_dev(hw)
    pwd = None if pw is None else to_dev(pw)
    normed = nrc.context_norms(xd, hwd, pwd, L, he, pe, hc, pc)
    kv_u = nrc.context_kv_project(normed, wd, split=split)
    h, r = nrc.context_hidden_norm(xd, hwd, pwd, L, he, pe, hc, pc)
    kv_f = nrc.context_kv_project_fused(h, r, pwd, wd, pc, split=split)
    torch.cuda.synchronize()
    return to_host(kv_u), to_host(kv_f)


@pytest.mark.parametrize("name", ["tiny", "prefill", "weightless", "long", "edge"])
def test_fused_project_parity_configs(nrc, oracle, name):
    """The fused projection at full size: bit-identical to the norms followed
    by the unfused projection (both GPU; the same MFMA accumulation order),
    and within the projection's tolerance of the oracle's FP32 sums of the
    oracle's norms on sampled rows (edge: every row whose norms are not all
    zero)."""
    cfg, d = _norms_inputs(name)
    _say(f"fused project {name}: L={cfg.L} T={cfg.T} N={cfg.N}")
    kv_u, kv_f = _fused_vs_unfused(nrc, d["x"], d["hidden_w"], d["pre_w"], d["w_kv"], cfg.L)
    assert_bits_equal(kv_f, kv_u, f"fused vs unfused {name}")
    del kv_u
    rng = np.random.default_rng(cfg.index + 7)
    n = min(cfg.T, 32)
    rows = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, n, replace=False)]))
    if cfg.edge:
        rows = np.unique(np.concatenate([rows[:2], _finite_edge_rows(d)]))
    on = oracle.context_norms(np.ascontiguousarray(d["x"][rows]), d["hidden_w"], d["pre_w"], cfg.L)
    ok, msg = projection_tolerance_ok(kv_f[:, rows], oracle.kv_project(on, d["w_kv"]))
    assert ok, f"fused {name}: {msg}"


@pytest.mark.parametrize("L,T,N", [(4, 16384, 128), (4, 16300, 128), (4, 16384, 256), (8, 8192, 128)])
def test_fused_project_narrow_heads(nrc, oracle, L, T, N):
    """A KV head or two per GPU at long-context sizes: the fused projection
    on 256 x 128 tiles (N = 128; a ragged last row tile at T = 16300) and in
    the layer-inner tile order (N <= 256) equals the norms followed by the
    unfused projection bit for bit, and is within tolerance of the oracle on
    sampled rows."""
    from norm_rope_cache_amd import synth

    lib = nrc._load()
    assert lib.nrc_context_kv_project_workspace_bytes(L, T, 8192, N) == 0, "shape should not split"
    x = synth.normal_bf16(7501 + T, (T, 8192))
    hw = synth.normal_bf16(7502, (8192,), 1.0, 0.3)
    pw = synth.normal_bf16(7503 + L, (L, 8192), 1.0, 0.3)
    w = synth.normal_bf16(7504 + N, (L, 8192, N), std=0.02)
    _say(f"fused narrow heads L={L} T={T} N={N}")
    kv_u, kv_f = _fused_vs_unfused(nrc, x, hw, pw, w, L)
    assert_bits_equal(kv_f, kv_u, f"fused vs unfused {L},{T},{N}")
    del kv_u
    rng = np.random.default_rng(T + N)
    rows = np.unique(np.concatenate([[0, 255, 256, T - 1], rng.choice(T, 24, replace=False)]))
    on = oracle.context_norms(np.ascontiguousarray(x[rows]), hw, pw, L)
    ok, msg = projection_tolerance_ok(kv_f[:, rows], oracle.kv_project(on, w))
    assert ok, f"fused narrow heads {L},{T},{N}: {msg}"


@pytest.mark.parametrize("L,T,N", [(4, 512, 1024), (2, 16, 128), (2, 300, 384), (3, 700, 512), (4, 256, 1024)])
def test_fused_split_matches_unfused_split(nrc, oracle, L, T, N):
    """The fused projection with its summation split (small T) equals the
    unfused split projection on the stacked norms bit for bit - the same
    slices and the same fixed-order addition - for 256 x 256 and 128 x 128
    slices, and is within tolerance of the oracle on sampled rows."""
    from norm_rope_cache_amd import synth

    lib = nrc._load()
    assert lib.nrc_context_kv_project_workspace_bytes(L, T, 8192, N) > 0, "shape should split"
    x = synth.normal_bf16(7401 + T, (T, 8192))
    hw = synth.normal_bf16(7402, (8192,), 1.0, 0.3)
    pw = synth.normal_bf16(7403, (L, 8192), 1.0, 0.3)
    w = synth.normal_bf16(7404 + N, (L, 8192, N), std=0.02)
    _say(f"fused split L={L} T={T} N={N}")
    kv_u, kv_f = _fused_vs_unfused(nrc, x, hw, pw, w, L, split=True)
    assert_bits_equal(kv_f, kv_u, f"fused split vs unfused split {L},{T},{N}")
    rows = np.unique(np.concatenate([[0, T - 1], np.arange(1, T, max(1, T // 20))]))
    on = oracle.context_norms(np.ascontiguousarray(x[rows]), hw, pw, L)
    ok, msg = projection_tolerance_ok(kv_f[:, rows], oracle.kv_project(on, w))
    assert ok, f"fused split {L},{T},{N}: {msg}"


def test_fused_split_special_values(nrc):
    """NaN / Inf / overflow / zero rows, -0.0 and NaN layer weights, non-zero
    centers, weightless layer norms: the fused split equals the unfused
    split bit for bit."""
    from norm_rope_cache_amd import synth

    T, L, N = 300, 3, 256
    x = synth.edge_mixture_bf16(191, 192, (T, 8192), nan_inf=True)
    x[3] = 0
    x[4] = 0x8000
    x[6, :] = 0x7F7F
    x[7:40] = synth.normal_bf16(194, (33, 8192))
    hw = synth.normal_bf16(195, (8192,), 1.0, 0.3)
    pw = synth.normal_bf16(196, (L, 8192), 1.0, 0.3)
    pw[:, ::83] = 0x8000
    pw_nan = pw.copy()
    pw_nan[2, 4000] = 0x7FC1
    w = synth.normal_bf16(197, (L, 8192, N), std=0.02)
    for pre_w, hc, pc in [(pw, 0.0, 0.0), (None, 0.0, 0.0), (pw, 0.5, -0.25), (pw_nan, 0.0, 0.0)]:
        _say(f"fused split specials pre_w={'yes' if pre_w is not None else 'no'} centers={hc},{pc}")
        kv_u, kv_f = _fused_vs_unfused(nrc, x, hw, pre_w, w, L, 1e-6, 1e-6, hc, pc, split=True)
        assert_bits_equal(kv_f, kv_u, f"fused split vs unfused split specials {hc},{pc}")


def test_fused_project_layer_changes_within_a_workgroup(nrc):
    """276 tiles of 256 x 256 over three layers (not a multiple of 8, so
    tiles go round-robin): the workgroups that take a second tile take it
    from another layer and restage its weight. Fused equals unfused bit for
    bit."""
    from norm_rope_cache_amd import synth

    L, T, N = 3, 5633, 1024
    x = synth.normal_bf16(7001, (T, 8192))
    hw = synth.normal_bf16(7002, (8192,), 1.0, 0.3)
    pw = synth.normal_bf16(7003, (L, 8192), 1.0, 0.3)
    w = synth.normal_bf16(7004, (L, 8192, N), std=0.02)
    _say(f"fused multi-tile L={L} T={T} N={N}")
    kv_u, kv_f = _fused_vs_unfused(nrc, x, hw, pw, w, L)
    assert_bits_equal(kv_f, kv_u, "fused vs unfused, several tiles per workgroup")


def test_fused_project_special_values(nrc):
    """NaN / Inf / overflow / zero rows (the exact-rounding rows of the fused
    path), -0.0 weights, weightless layer norms and non-zero centers: fused
    and unfused projections agree bit for bit."""
    from norm_rope_cache_amd import synth

    T, L, N = 300, 3, 256
    x = synth.edge_mixture_bf16(91, 92, (T, 8192), nan_inf=True)
    x[3] = 0
    x[4] = 0x8000
    x[5] = synth.normal_bf16(93, (8192,))
    x[6, :] = 0x7F7F
    x[7:40] = synth.normal_bf16(94, (33, 8192))
    hw = synth.normal_bf16(95, (8192,), 1.0, 0.3)
    hw[::101] = 0x8000
    pw = synth.normal_bf16(96, (L, 8192), 1.0, 0.3)
    pw[:, ::83] = 0x8000
    w = synth.normal_bf16(97, (L, 8192, N), std=0.02)
    for pre_w, hc, pc in [(pw, 0.0, 0.0), (None, 0.0, 0.0), (pw, 0.5, -0.25), (pw, -0.0, -0.0), (pw, 0.0, 0.0)]:
        wts = pre_w
        _say(f"fused specials pre_w={'yes' if wts is not None else 'no'} centers={hc},{pc}")
        kv_u, kv_f = _fused_vs_unfused(nrc, x, hw, wts, w, L, 1e-6, 1e-6, hc, pc)
        assert_bits_equal(kv_f, kv_u, f"fused vs unfused specials {hc},{pc}")
    # a NaN layer weight forces the exact rounding on every row
    pw_nan = pw.copy()
    pw_nan[1, 17] = 0x7FC1
    kv_u, kv_f = _fused_vs_unfused(nrc, x, hw, pw_nan, w, L)
    assert_bits_equal(kv_f, kv_u, "fused vs unfused with a NaN layer weight")


def test_fused_chain_matches_unfused_chain(nrc):
    """context_kv_chain fused and unfused (one-pass projection) write
    identical caches."""
    from norm_rope_cache_amd import synth

    cfg = synth.scaled(synth.PREFILL, 200)
    d = synth.make_inputs(cfg, with_cache=True)
    outs = []
    for fused in (True, False):
        cd = to_dev(d["caches"])
        kv = nrc.context_kv_chain(to_dev(d["x"]), to_dev(d["hidden_w"]), to_dev(d["pre_w"]), to_dev(d["w_kv"]),
                                  to_dev(d["positions"]), to_dev(d["slots"]), to_dev(d["cos_sin"]), cd, cfg.H,
                                  fused=fused, split=False)
        outs.append((to_host(kv), to_host(cd)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])
