"""Seeded synthetic inputs for the context K/V chain.

One generator serves the tests, the bench and the smoke check; both the HIP
path and the CPU oracle receive the arrays it returns. It holds none of the
chain's arithmetic: it only draws numbers.

Recipe (documented in the design notes):
  * SplitMix64 (Vigna's public-domain mixer): output i of a stream with seed s
    is mix(s + (i + 1) * 0x9E3779B97F4A7C15) mod 2^64.
  * uniform doubles in [0, 1): top 53 bits of an output times 2^-53.
  * normals: Box-Muller in double on consecutive uniform pairs (both the cos
    and the sin branch), then float32 (numpy) and bf16 (torch's conversion).
  * config i (1..5) has seed 0x6E72630000 + i; tensor `tid` of a config draws
    from the stream seed * 64 + tid.
bf16 tensors are numpy uint16 arrays holding the bit patterns.
"""

import os
from dataclasses import dataclass

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
CHUNK = 1 << 22

D = 8192
HEAD_DIM = 64

# tensor ids of a config's streams
TID_X, TID_HW, TID_PW, TID_W, TID_POS, TID_SLOT, TID_NEG, TID_BLOCKS = 1, 2, 3, 4, 5, 6, 7, 8
TID_CACHE, TID_MIX, TID_ZROWS, TID_KV, TID_KVMIX, TID_BASE = 9, 10, 11, 12, 13, 14


def splitmix64(seed, n, start=0):
    """Outputs start .. start+n-1 of the SplitMix64 stream `seed` (uint64)."""
    seed = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = seed + idx * GOLDEN
        z ^= z >> np.uint64(30)
        z *= M1
        z ^= z >> np.uint64(27)
        z *= M2
        z ^= z >> np.uint64(31)
    return z


def uniform(seed, n, start=0):
    """Doubles in [0, 1)."""
    return (splitmix64(seed, n, start) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def _normal_pairs(seed, p0, p1):
    """Normals 2*p0 .. 2*p1-1 of stream `seed` (float64)."""
    u = uniform(seed, 2 * (p1 - p0), 2 * p0)
    u1 = 1.0 - u[0::2]  # (0, 1]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    th = 2.0 * np.pi * u2
    z = np.empty(2 * (p1 - p0), dtype=np.float64)
    z[0::2] = r * np.cos(th)
    z[1::2] = r * np.sin(th)
    return z


def normal(seed, n):
    """n standard normals (float64), Box-Muller over pairs of uniforms."""
    out = np.empty(n, dtype=np.float64)
    pairs = (n + 1) // 2
    for p0 in range(0, pairs, CHUNK):
        p1 = min(pairs, p0 + CHUNK)
        z = _normal_pairs(seed, p0, p1)
        lo, hi = 2 * p0, min(n, 2 * p1)
        out[lo:hi] = z[: hi - lo]
    return out


def to_bf16_bits(a):
    """float array -> bf16 bit patterns (uint16) through torch's conversion."""
    import torch

    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _pool_map(fn, starts):
    """Run fn over chunk starts on a few threads (numpy releases the GIL);
    each chunk depends only on its start, so the result is order-free."""
    from concurrent.futures import ThreadPoolExecutor

    workers = max(1, min(8, (os.cpu_count() or 1)))
    if len(starts) <= 1 or workers == 1:
        for s0 in starts:
            fn(s0)
        return
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fn, starts))


def normal_bf16(seed, shape, mean=0.0, std=1.0):
    """bf16 bits of mean + std * N(0, 1), drawn in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    pairs = (n + 1) // 2

    def one(p0):
        p1 = min(pairs, p0 + CHUNK)
        z = _normal_pairs(seed, p0, p1)
        lo, hi = 2 * p0, min(n, 2 * p1)
        out[lo:hi] = to_bf16_bits(mean + std * z[: hi - lo])

    _pool_map(one, list(range(0, pairs, CHUNK)))
    return out.reshape(shape)


def normal_f32(seed, shape, mean=0.0, std=1.0):
    """float32 values of mean + std * N(0, 1) (FP32 norm weights)."""
    n = int(np.prod(shape))
    return (mean + std * normal(seed, n)).astype(np.float32).reshape(shape)


def random_bits_u16(seed, shape):
    """Uniform random 16-bit patterns (e.g. a cache's prior contents)."""
    n = int(np.prod(shape))
    words = (n + 3) // 4
    z = np.empty(words, dtype=np.uint64)

    def one(i0):
        i1 = min(words, i0 + CHUNK)
        z[i0:i1] = splitmix64(seed, i1 - i0, i0)

    _pool_map(one, list(range(0, words, CHUNK)))
    return z.view(np.uint16)[:n].reshape(shape)


def bf16_bits_range(seed, shape, emin=-6):
    """Random bf16 bit patterns built directly (no rounding): random sign,
    exponent uniform in [emin, emin + 7], random 7-bit mantissa. A fast
    stand-in for large activation tensors."""
    n = int(np.prod(shape))
    out = random_bits_u16(seed, (n,))
    base = np.uint16((emin + 127) << 7)

    def one(i0):
        v = out[i0:i0 + 4 * CHUNK]
        e = (v >> np.uint16(7)) & np.uint16(7)
        v &= np.uint16(0x807F)
        v |= (e << np.uint16(7)) + base

    _pool_map(one, list(range(0, n, 4 * CHUNK)))
    return out.reshape(shape)


def permutation(seed, n):
    """A seeded permutation of 0..n-1 (argsort of random keys, stable)."""
    return np.argsort(splitmix64(seed, n), kind="stable").astype(np.int64)


def rope_table(max_position, base=10000.0):
    """bf16 [max_position, 64]: row p = cos(p theta_j) for j < 32, then
    sin(p theta_j), theta_j = base^(-2j/64); angles and cos/sin in double."""
    j = np.arange(HEAD_DIM // 2, dtype=np.float64)
    theta = base ** (-2.0 * j / HEAD_DIM)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * theta[None, :]
    tab = np.concatenate([np.cos(ang), np.sin(ang)], axis=1)
    return to_bf16_bits(tab).reshape(max_position, HEAD_DIM)


def edge_mixture_bf16(seed_mix, seed_normal, shape, nan_inf=False):
    """Per element, i.i.d.: 1% -0.0; 1% bf16 subnormal (random sign, mantissa
    1..127); 0.1% near the bf16 maximum (random sign, one of the 16 largest
    finite magnitudes 0x7F70..0x7F7F); the rest N(0, 1). With nan_inf, a
    further 0.05% are +-Inf and 0.05% NaN."""
    n = int(np.prod(shape))
    out = normal_bf16(seed_normal, (n,))
    u = uniform(seed_mix, n)
    bits = splitmix64(seed_mix + 1, n)
    sign = ((bits >> np.uint64(63)).astype(np.uint16) << np.uint16(15)).astype(np.uint16)
    low7 = ((bits & np.uint64(0x7F)).astype(np.uint16))
    sub = np.where(low7 == 0, np.uint16(1), low7).astype(np.uint16)
    big = (np.uint16(0x7F70) + (bits >> np.uint64(8) & np.uint64(0xF)).astype(np.uint16)).astype(np.uint16)
    m_neg0 = u < 0.01
    m_sub = (u >= 0.01) & (u < 0.02)
    m_big = (u >= 0.02) & (u < 0.021)
    out[m_neg0] = np.uint16(0x8000)
    out[m_sub] = sign[m_sub] | sub[m_sub]
    out[m_big] = sign[m_big] | big[m_big]
    if nan_inf:
        m_inf = (u >= 0.021) & (u < 0.0215)
        m_nan = (u >= 0.0215) & (u < 0.022)
        out[m_inf] = sign[m_inf] | np.uint16(0x7F80)
        out[m_nan] = np.uint16(0x7FC1) | sign[m_nan]
    return out.reshape(shape)


@dataclass(frozen=True)
class Config:
    name: str
    index: int  # 1..5
    L: int
    T: int
    H: int
    block_size: int
    num_blocks: int
    max_position: int  # 0: RoPE off
    hidden_weighted: bool = True
    pre_weighted: bool = True
    x_std: float = 1.0
    edge: bool = False

    @property
    def N(self):
        return 2 * self.H * HEAD_DIM

    @property
    def rope(self):
        return self.max_position > 0

    @property
    def seed(self):
        return 0x6E72630000 + self.index

    def stream(self, tid):
        return self.seed * 64 + tid


TINY = Config("tiny", 1, L=2, T=16, H=1, block_size=16, num_blocks=4, max_position=4096)
PREFILL = Config("prefill", 2, L=4, T=512, H=8, block_size=16, num_blocks=2048, max_position=32768)
WEIGHTLESS = Config("weightless", 3, L=4, T=4096, H=8, block_size=32, num_blocks=4096, max_position=0,
                    hidden_weighted=False, x_std=2.0)
LONG = Config("long", 4, L=4, T=16384, H=8, block_size=16, num_blocks=8192, max_position=131072)
EDGE = Config("edge", 5, L=8, T=32768, H=16, block_size=64, num_blocks=1024, max_position=131072, edge=True)

CONFIGS = {c.name: c for c in (TINY, PREFILL, WEIGHTLESS, LONG, EDGE)}


def scaled(cfg, T, num_blocks=None, name=None):
    """The same recipe at another row count (parity cases the oracle finishes
    in seconds); slot-space and block size stay, the block count may shrink."""
    from dataclasses import replace

    return replace(cfg, name=name or f"{cfg.name}_T{T}", T=T, num_blocks=num_blocks or cfg.num_blocks)


def positions(cfg):
    T = cfg.T
    if cfg.name.startswith("tiny") or cfg.name.startswith("long"):
        pos = np.arange(T, dtype=np.int64)
        if cfg.max_position:
            pos %= cfg.max_position
        return pos
    hi = cfg.max_position if cfg.max_position else 32768
    return np.minimum((uniform(cfg.stream(TID_POS), T) * hi).astype(np.int64), hi - 1)


def slot_mapping(cfg):
    """int64 [T] slots shared by every layer, per config recipe."""
    T, n_slots = cfg.T, cfg.num_blocks * cfg.block_size
    kind = cfg.name.split("_")[0]
    if kind == "tiny":
        s = permutation(cfg.stream(TID_SLOT), n_slots)[:T].copy()
        neg = permutation(cfg.stream(TID_NEG), T)[:2]
        s[neg] = -1
        return s
    if kind == "prefill":
        s = permutation(cfg.stream(TID_SLOT), n_slots)[:T].copy()
        neg = permutation(cfg.stream(TID_NEG), T)[: int(round(0.05 * T))]
        s[neg] = -1
        return s
    if kind == "weightless":
        base = int(uniform(cfg.stream(TID_BASE), 1)[0] * (n_slots - T + 1))
        return base + np.arange(T, dtype=np.int64)
    if kind == "long":
        bs = cfg.block_size
        nblk = (T + bs - 1) // bs
        table = permutation(cfg.stream(TID_BLOCKS), cfg.num_blocks)[:nblk]
        t = np.arange(T, dtype=np.int64)
        return table[t // bs] * bs + t % bs
    if kind == "edge":
        s = np.full(T, -1, dtype=np.int64)
        valid = np.sort(permutation(cfg.stream(TID_NEG), T)[T // 2:])
        s[valid] = permutation(cfg.stream(TID_SLOT), n_slots)[: valid.size]
        return s
    raise ValueError(cfg.name)


def make_inputs(cfg, with_cache=True, kv_synth=False, with_x=True, with_weights=True):
    """All operands of one config (numpy, bf16 as uint16 bits).

    Returns a dict with x, hidden_w, pre_w, w_kv, cos_sin, positions, slots
    ([L, T], one shared mapping), eps values, and (with_cache) caches
    [L, num_blocks, H, block_size, 128] pre-filled with random bits. With
    kv_synth, also `kv`: a synthetic projection output [L, T, N] of the
    projection's scale (N(0, 1.8); for the edge config the edge mixture with
    NaN and Inf) to drive the store on its own."""
    L, T, H, N = cfg.L, cfg.T, cfg.H, cfg.N
    out = {"cfg": cfg, "hidden_eps": 1e-6, "pre_eps": 1e-6, "k_eps": 1e-6}
    if not with_x:
        pass
    elif cfg.edge:
        x = edge_mixture_bf16(cfg.stream(TID_MIX), cfg.stream(TID_X), (T, D))
        nz = max(1, int(round(0.01 * T)))
        zrows = permutation(cfg.stream(TID_ZROWS), T)[:nz]
        x[zrows] = 0
        out["zero_rows"] = np.sort(zrows)
    else:
        x = normal_bf16(cfg.stream(TID_X), (T, D), std=cfg.x_std)
    if with_x:
        out["x"] = x
    if with_weights:
        out["hidden_w"] = normal_bf16(cfg.stream(TID_HW), (D,), mean=1.0, std=0.1) if cfg.hidden_weighted else None
        out["pre_w"] = normal_bf16(cfg.stream(TID_PW), (L, D), mean=1.0, std=0.1) if cfg.pre_weighted else None
        out["w_kv"] = normal_bf16(cfg.stream(TID_W), (L, D, N), std=0.02)
    out["cos_sin"] = rope_table(cfg.max_position) if cfg.rope else None
    out["positions"] = positions(cfg)
    s = slot_mapping(cfg)
    out["slots"] = np.ascontiguousarray(np.broadcast_to(s, (L, T)))
    if with_cache:
        out["caches"] = random_bits_u16(cfg.stream(TID_CACHE), (L, cfg.num_blocks, H, cfg.block_size, 2 * HEAD_DIM))
    if kv_synth:
        if cfg.edge:
            out["kv"] = edge_mixture_bf16(cfg.stream(TID_KVMIX), cfg.stream(TID_KV), (L, T, N), nan_inf=True)
        else:
            out["kv"] = normal_bf16(cfg.stream(TID_KV), (L, T, N), std=1.8)
    return out
