"""Pins that tie the CPU oracle to something other than itself.

Each pin takes the oracle module and raises AssertionError when the oracle
disagrees with the pages' worked examples, a closed form, an invariant of the
paged layout, or a pure-Python brute force written here from the textbook
definition.  tests/test_oracle_pins.py runs every pin, and runs them all again
against deliberately broken copies of oracle functions to show that each
plausible mistake is caught by at least one pin.
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- helpers (independent of the oracle)

def bf16_value(pattern: int) -> float:
    return struct.unpack(">f", struct.pack(">I", (int(pattern) & 0xFFFF) << 16))[0]


def brute_force(q, K, V, scale):
    """Textbook softmax(q K^T scale) V with Python floats.

    q: [H][D]; K, V: [L][H][D] (a never-paged, contiguous cache).  Sums use
    math.fsum, so the result is accurate to a few float64 ulps.
    """
    L, H, D = len(K), len(q), len(q[0])
    out = []
    for h in range(H):
        s = [scale * math.fsum(q[h][d] * K[t][h][d] for d in range(D)) for t in range(L)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        z = math.fsum(w)
        out.append([math.fsum(w[t] * V[t][h][d] for t in range(L)) / z for d in range(D)])
    return out


def place(logical, table, bs, pool):
    """Scatter a contiguous [L, H, D] cache into pool [NB, H, bs, D] through ``table``.

    Written element by element from the layout's definition: logical token t
    sits in physical block table[t // bs] at offset t % bs.
    """
    L, H, D = logical.shape
    for t in range(L):
        b = table[t // bs]
        for h in range(H):
            pool[b, h, t % bs, :] = logical[t, h, :]


class Case:
    """A small random paged decode problem built from contiguous K/V."""

    def __init__(self, rng, lens, H, D, bs, dtype="f32", pool_extra=5, scale=None, poison=True):
        self.lens, self.H, self.D, self.bs, self.dtype = list(lens), H, D, bs, dtype
        nblk = [-(-L // bs) for L in lens]
        NB = sum(nblk) + pool_extra
        perm = rng.permutation(NB)
        M = max(nblk) + 2
        self.tables = np.full((len(lens), M), -1, dtype=np.int32)
        pos = 0
        for i, n in enumerate(nblk):
            self.tables[i, :n] = perm[pos:pos + n]
            pos += n
        self.scale = (1.0 / math.sqrt(D)) if scale is None else scale
        B = len(lens)
        if dtype == "f32":
            self.q = rng.standard_normal((B, H, D)).astype(np.float32)
            self.Klog = [rng.standard_normal((L, H, D)).astype(np.float32) for L in lens]
            self.Vlog = [rng.standard_normal((L, H, D)).astype(np.float32) for L in lens]
            fill = np.float32(np.nan) if poison else np.float32(0)
            self.k_pool = np.full((NB, H, bs, D), fill, dtype=np.float32)
            self.v_pool = np.full((NB, H, bs, D), fill, dtype=np.float32)
            to_py = float
        elif dtype == "bf16":
            def bits(shape):
                x = rng.standard_normal(shape).astype(np.float32)
                return (x.view(np.uint32) >> 16).astype(np.uint16)      # truncated bf16 patterns
            self.q = bits((B, H, D))
            self.Klog = [bits((L, H, D)) for L in lens]
            self.Vlog = [bits((L, H, D)) for L in lens]
            fill = np.uint16(0x7FC0) if poison else np.uint16(0)          # bf16 quiet NaN
            self.k_pool = np.full((NB, H, bs, D), fill, dtype=np.uint16)
            self.v_pool = np.full((NB, H, bs, D), fill, dtype=np.uint16)
            to_py = bf16_value
        elif dtype == "f16":
            self.q = rng.standard_normal((B, H, D)).astype(np.float16)
            self.Klog = [rng.standard_normal((L, H, D)).astype(np.float16) for L in lens]
            self.Vlog = [rng.standard_normal((L, H, D)).astype(np.float16) for L in lens]
            fill = np.float16(np.nan) if poison else np.float16(0)
            self.k_pool = np.full((NB, H, bs, D), fill, dtype=np.float16)
            self.v_pool = np.full((NB, H, bs, D), fill, dtype=np.float16)
            to_py = float
        else:
            raise ValueError(dtype)
        self.to_py = to_py
        for i in range(B):
            place(self.Klog[i], self.tables[i], bs, self.k_pool)
            place(self.Vlog[i], self.tables[i], bs, self.v_pool)
        self.context_lens = np.array(lens, dtype=np.int32)

    def expected(self, i):
        f = self.to_py
        q = [[f(x) for x in row] for row in self.q[i]]
        K = [[[f(x) for x in r] for r in tok] for tok in self.Klog[i]]
        V = [[[f(x) for x in r] for r in tok] for tok in self.Vlog[i]]
        return np.array(brute_force(q, K, V, self.scale))

    def run(self, o, **kw):
        return o.decode(self.q, self.k_pool, self.v_pool, self.tables, self.context_lens, self.scale,
                        self.bs, self.dtype, **kw)


# ---------------------------------------------------------------- pins

def pin_block_counts(o):
    g = golden("block_counts.json")
    bs = g["block_size"]
    for n, nb in g["blocks"]:
        assert o.blocks_needed(n, bs) == nb, (n, o.blocks_needed(n, bs), nb)
    for n, empty in g["empty_slots"]:
        assert o.blocks_needed(n, bs) * bs - n == empty
    fr = g["four_requests"]
    assert sum(o.blocks_needed(n, bs) for n in fr["lens"]) == fr["total_blocks"]
    worst = max(o.blocks_needed(n, bs) * bs - n for n in range(1, 10 * bs))
    assert worst == g["max_empty_slots"]


def pin_storage_upcast(o):
    g = golden("storage_bits.json")
    for h, v in g["bf16"]:
        got = o.to_float64(np.array([int(h, 16)], dtype=np.uint16), "bf16")[0]
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (h, got, v)
    for h, v in g["f16"]:
        got = o.to_float64(np.array([int(h, 16)], dtype=np.uint16), "f16")[0]
        assert got == v, (h, got, v)
    x = np.float32(1.0 / 3.0)
    assert o.to_float64(np.array([x]), "f32")[0] == float(x)


def pin_slot_example(o):
    g = golden("slot_example.json")
    bs, blk = g["block_size"], g["block"]
    assert o.slot_to_block_offset(g["decode_flat_slot"], bs) == (blk, g["decode_offset"])
    for off in g["prompt_offsets"]:
        assert o.slot_to_block_offset(blk * bs + off, bs) == (blk, off)
    rng = np.random.default_rng(7)
    H, D, NB = 2, 8, 64
    k_pool = rng.integers(0, 2 ** 16, (NB, H, bs, D), dtype=np.uint16)
    v_pool = rng.integers(0, 2 ** 16, (NB, H, bs, D), dtype=np.uint16)
    k = rng.integers(0, 2 ** 16, (3, H, D), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, (3, H, D), dtype=np.uint16)
    slots = np.array([g["decode_flat_slot"], -1, 5 * bs + 15], dtype=np.int64)
    before = k_pool.copy()
    k2, v2 = o.kv_write(k, v, slots, k_pool, v_pool, bs)
    assert np.array_equal(k_pool, before)                     # inputs are not modified in place
    exp_k, exp_v = k_pool.copy(), v_pool.copy()
    exp_k[blk, :, g["decode_offset"], :] = k[0]
    exp_v[blk, :, g["decode_offset"], :] = v[0]
    exp_k[5, :, 15, :] = k[2]
    exp_v[5, :, 15, :] = v[2]
    assert np.array_equal(k2, exp_k) and np.array_equal(v2, exp_v)


def pin_write_then_read(o):
    """Writing a sequence token by token through its slots, then gathering, returns it in order."""
    rng = np.random.default_rng(11)
    bs, H, D, NB = 16, 3, 8, 40
    table = rng.permutation(NB)[:4]
    L = 53
    toks = (rng.integers(0, 0x7F80, (L, H, D)) | (rng.integers(0, 2, (L, H, D)) << 15)).astype(np.uint16)
    k_pool = np.full((NB, H, bs, D), 0x7FC0, dtype=np.uint16)
    v_pool = np.full((NB, H, bs, D), 0x7FC0, dtype=np.uint16)
    slots = np.array([int(table[t // bs]) * bs + t % bs for t in range(L)], dtype=np.int64)
    k_pool, v_pool = o.kv_write(toks, toks[::-1].copy(), slots, k_pool, v_pool, bs)
    back = o.gather_sequence(k_pool, table, L, bs, "bf16")
    assert np.array_equal(back, o.to_float64(toks, "bf16").transpose(1, 0, 2))
    backv = o.gather_sequence(v_pool, table, L, bs, "bf16")
    assert np.array_equal(backv, o.to_float64(toks[::-1], "bf16").transpose(1, 0, 2))


def pin_write_bitwise(o):
    """The write moves stored bits: NaN payloads and -0.0 survive unchanged."""
    bs, H, D, NB = 16, 1, 4, 4
    k = np.array([[[0x7FC1, 0x8000, 0xFF81, 0x0001]]], dtype=np.uint16)
    pool = np.zeros((NB, H, bs, D), dtype=np.uint16)
    k2, v2 = o.kv_write(k, k, np.array([2 * bs + 3]), pool, pool, bs)
    assert np.array_equal(k2[2, 0, 3], k[0, 0]) and np.array_equal(v2[2, 0, 3], k[0, 0])
    f = np.array([[[np.float32(-0.0), np.float32(np.nan), 1.5, -2.0]]], dtype=np.float32)
    poolf = np.ones((NB, H, bs, D), dtype=np.float32)
    k3, _ = o.kv_write(f, f, np.array([7]), poolf, poolf, bs)
    assert np.array_equal(k3[0, 0, 7].view(np.uint32), f[0, 0].view(np.uint32))


def pin_brute_force(o):
    """The paged oracle equals the textbook formula on never-paged K/V."""
    rng = np.random.default_rng(1234)
    cases = [
        Case(rng, [6, 50, 8, 100], H=4, D=64, bs=16),                      # the pages' four requests
        Case(rng, [1, 16, 17, 33], H=2, D=8, bs=16, scale=0.37),
        Case(rng, [31, 5, 64], H=3, D=16, bs=32, dtype="bf16"),
        Case(rng, [2, 40], H=2, D=4, bs=16, scale=2.5),
    ]
    for c in cases:
        got = c.run(o)
        for i in range(len(c.lens)):
            exp = c.expected(i)
            assert np.max(np.abs(got[i] - exp)) <= 1e-12 * max(1.0, np.max(np.abs(exp))), (c.lens, i)


def pin_pages_tables(o):
    """The pages' example tables, read in place, give the textbook result."""
    g = golden("tables.json")
    rng = np.random.default_rng(5)
    H, D, bs = 2, 8, 16
    tabs = [g["card"]["table"], g["step5_request_b"]["table"]] + list(g["memory_usage"]["tables"].values())
    lens = [40, 35, 9, 37, 16]
    NB = 100
    B = len(tabs)
    tables = np.full((B, 4), -1, dtype=np.int32)
    k_pool = np.full((NB, H, bs, D), np.nan, dtype=np.float32)
    v_pool = np.full((NB, H, bs, D), np.nan, dtype=np.float32)
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    Ks, Vs = [], []
    assert len(set(sum(tabs, []))) == sum(len(t) for t in tabs)      # the examples' ids are disjoint
    for i, (t, L) in enumerate(zip(tabs, lens)):
        assert len(t) == -(-L // bs)
        tables[i, :len(t)] = t
        K = rng.standard_normal((L, H, D)).astype(np.float32)
        V = rng.standard_normal((L, H, D)).astype(np.float32)
        place(K, t, bs, k_pool)
        place(V, t, bs, v_pool)
        Ks.append(K)
        Vs.append(V)
    lens_a = np.array(lens, dtype=np.int32)
    got = o.decode(q, k_pool, v_pool, tables, lens_a, 0.5, bs, "f32")
    for i in range(B):
        exp = np.array(brute_force(q[i].astype(float).tolist(), Ks[i].astype(float).tolist(),
                                   Vs[i].astype(float).tolist(), 0.5))
        assert np.max(np.abs(got[i] - exp)) <= 1e-12


def pin_permutation_invariance(o):
    """Relabelling physical blocks (moving them and rewriting tables) changes nothing, bit for bit."""
    rng = np.random.default_rng(99)
    c = Case(rng, [6, 50, 8, 100, 1], H=4, D=16, bs=16, pool_extra=20)
    base = c.run(o)
    NB = c.k_pool.shape[0]
    for _ in range(3):
        pi = rng.permutation(NB)
        kp = np.empty_like(c.k_pool)
        vp = np.empty_like(c.v_pool)
        kp[pi] = c.k_pool
        vp[pi] = c.v_pool
        tabs = np.where(c.tables >= 0, pi[np.maximum(c.tables, 0)], -1).astype(np.int32)
        got = o.decode(c.q, kp, vp, tabs, c.context_lens, c.scale, c.bs, c.dtype)
        assert np.array_equal(got, base)


def pin_poison_invariance(o):
    """Slots past L, blocks in no table and table padding never reach the output."""
    rng = np.random.default_rng(3)
    clean = Case(np.random.default_rng(3), [6, 50, 8, 100], H=2, D=8, bs=16, poison=False)
    dirty = Case(rng, [6, 50, 8, 100], H=2, D=8, bs=16, poison=True)
    a, b = clean.run(o), dirty.run(o)
    assert np.all(np.isfinite(b)) and np.array_equal(a, b)
    tabs = dirty.tables.copy()
    tabs[tabs < 0] = 10 ** 6                       # padding that would be out of range if read
    c = o.decode(dirty.q, dirty.k_pool, dirty.v_pool, tabs, dirty.context_lens, dirty.scale, 16, "f32")
    assert np.array_equal(c, b)


def pin_closed_forms(o):
    rng = np.random.default_rng(21)
    bs, H, D = 16, 3, 8
    # one token: the output is that token's V row exactly
    c = Case(rng, [1, 1], H=H, D=D, bs=bs, scale=1.7)
    got = c.run(o)
    for i in range(2):
        assert np.array_equal(got[i], c.Vlog[i][0].astype(np.float64))
    # q = 0 (or scale = 0): the mean of V over the context
    c = Case(rng, [37, 5], H=H, D=D, bs=bs)
    c.q[:] = 0
    got = c.run(o)
    for i in range(2):
        assert np.allclose(got[i], c.Vlog[i].astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)
    # a constant V row is returned unchanged
    c = Case(rng, [29], H=H, D=D, bs=bs)
    c.Vlog[0][:] = np.float32(0.625)
    place(c.Vlog[0], c.tables[0], bs, c.v_pool)
    assert np.allclose(c.run(o)[0], 0.625, rtol=0, atol=1e-15)
    # two tokens: sigmoid weights
    c = Case(rng, [2], H=1, D=4, bs=bs, scale=0.8)
    q = c.q[0, 0].astype(float)
    k0, k1 = c.Klog[0][0, 0].astype(float), c.Klog[0][1, 0].astype(float)
    v0, v1 = c.Vlog[0][0, 0].astype(float), c.Vlog[0][1, 0].astype(float)
    s0, s1 = 0.8 * math.fsum(q * k0), 0.8 * math.fsum(q * k1)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert np.allclose(c.run(o)[0, 0], w0 * v0 + (1 - w0) * v1, rtol=0, atol=1e-14)
    # hand example: scores 1, 0, -1 -> weights e, 1, 1/e
    q = np.array([[[1, 0]]], dtype=np.float32)
    kp = np.zeros((2, 1, bs, 2), dtype=np.float32)
    vp = np.zeros((2, 1, bs, 2), dtype=np.float32)
    kp[1, 0, :3] = [[1, 0], [0, 1], [-1, 0]]
    vp[1, 0, :3] = [[1, 0], [0, 1], [0, 0]]
    got = o.decode(q, kp, vp, np.array([[1]], dtype=np.int32), np.array([3]), 1.0, bs, "f32")
    z = math.e + 1 + 1 / math.e
    assert np.allclose(got[0, 0], [math.e / z, 1 / z], rtol=0, atol=1e-15)
    # linearity in V and scale folding
    c = Case(rng, [45, 17], H=H, D=D, bs=bs)
    a = c.run(o)
    c2 = Case(np.random.default_rng(0), [45, 17], H=H, D=D, bs=bs)
    c2.q, c2.k_pool, c2.tables, c2.scale = c.q, c.k_pool, c.tables, c.scale
    c.v_pool = (np.round(c.v_pool * 256) / 256).astype(np.float32)      # exact under the maps below
    a = c.run(o)
    c2.v_pool = np.where(np.isnan(c.v_pool), np.nan, -2.0 * c.v_pool + 0.5).astype(np.float32)
    assert np.allclose(c2.run(o), -2.0 * a + 0.5, rtol=0, atol=1e-12)
    c3 = Case(np.random.default_rng(0), [45, 17], H=H, D=D, bs=bs)
    c3.q, c3.k_pool, c3.v_pool, c3.tables = c.q * np.float32(2.0), c.k_pool, c.v_pool, c.tables
    c3.scale = c.scale / 2.0
    assert np.allclose(c3.run(o), a, rtol=0, atol=1e-13)
    # empty context: zero row
    c = Case(rng, [4, 9], H=H, D=D, bs=bs)
    c.context_lens[0] = 0
    got = c.run(o)
    assert np.array_equal(got[0], np.zeros((H, D)))


def pin_split_equals_single(o):
    """Partitioned evaluation with a log-sum-exp merge equals the one-pass result."""
    rng = np.random.default_rng(8)
    for lens, bs, parts in (([6, 50, 8, 100], 16, (16, 32, 48, 512)),
                            ([700, 33, 1024], 16, (64, 256, 512)),
                            ([95, 400], 32, (32, 64, 128))):
        c = Case(rng, lens, H=2, D=8, bs=bs)
        one = c.run(o)
        for P in parts:
            sp = o.decode_split(c.q, c.k_pool, c.v_pool, c.tables, c.context_lens, c.scale, bs, c.dtype, P)
            assert np.max(np.abs(sp - one)) <= 1e-12, (lens, P)
    # widely different partition maxima still merge correctly
    c = Case(rng, [64], H=1, D=4, bs=16, scale=1.0)
    c.Klog[0][:32] *= 30
    place(c.Klog[0], c.tables[0], 16, c.k_pool)
    ref = c.expected(0)
    sp = o.decode_split(c.q, c.k_pool, c.v_pool, c.tables, c.context_lens, 1.0, 16, "f32", 16)
    assert np.max(np.abs(sp[0] - ref)) <= 1e-12


def pin_prefix_sharing(o):
    """Tables that share a physical block equal the same data duplicated into private blocks."""
    g = golden("tables.json")["prefix_sharing"]
    rng = np.random.default_rng(4)
    bs, H, D, NB = 16, 2, 8, 80
    tabs = list(g["tables"].values())
    shared = g["shared_block"]
    lens = [bs + 3, bs + 11, bs + 16]
    k_pool = rng.standard_normal((NB, H, bs, D)).astype(np.float32)
    v_pool = rng.standard_normal((NB, H, bs, D)).astype(np.float32)
    q = rng.standard_normal((3, H, D)).astype(np.float32)
    tables = np.array(tabs, dtype=np.int32)
    a = o.decode(q, k_pool, v_pool, tables, np.array(lens), 0.3, bs, "f32")
    private = [70, 71, 72]
    tables2 = tables.copy()
    for i, p in enumerate(private):
        k_pool[p] = k_pool[shared]
        v_pool[p] = v_pool[shared]
        tables2[i, 0] = p
    b = o.decode(q, k_pool, v_pool, tables2, np.array(lens), 0.3, bs, "f32")
    assert np.array_equal(a, b)


def pin_newest_token_slots(o):
    """The pages' block 42: after the 6-token prompt and one decode token the newest token (the 7th)
    sits in slot 6 (flat 678); the 16th fills slot 15; the 17th opens the table's second block."""
    g = golden("slot_example.json")
    bs = g["block_size"]
    tables = np.array([[42, 9], [42, 9], [42, 9], [5, -1], [42, 9]], dtype=np.int32)
    lens = np.array([7, 16, 17, 0, 1])
    got = o.newest_token_slots(tables, lens, bs).tolist()
    assert got == [g["decode_flat_slot"], 42 * bs + 15, 9 * bs, -1, 42 * bs]
    # agrees with where a write of the newest token makes the gather find it
    rng = np.random.default_rng(24)
    c = Case(rng, [3, 16, 17, 40], H=2, D=4, bs=bs)
    s = o.newest_token_slots(c.tables, c.context_lens, bs)
    for i, L in enumerate(c.lens):
        b, off = o.slot_to_block_offset(int(s[i]), bs)
        assert np.array_equal(c.k_pool[b, :, off, :], c.Klog[i][L - 1])


def _prefill_case(rng, lens, news, H=2, D=8, bs=16, dtype="f32"):
    """A Case whose sequence i holds lens[i] tokens, the last news[i] of them new (with queries)."""
    c = Case(rng, lens, H=H, D=D, bs=bs, dtype=dtype)
    qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    if dtype == "f32":
        q = rng.standard_normal((int(qs[-1]), H, D)).astype(np.float32)
    else:
        q = (rng.standard_normal((int(qs[-1]), H, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return c, q, qs


def pin_prefill_brute_force(o):
    """Every query row against textbook softmax over the tokens up to and including its own position."""
    rng = np.random.default_rng(25)
    for dtype in ("f32", "bf16"):
        c, q, qs = _prefill_case(rng, [6, 20, 37], [6, 4, 37], dtype=dtype)
        got = o.prefill(q, c.k_pool, c.v_pool, c.tables, qs, c.context_lens, c.scale, c.bs, dtype)
        f = c.to_py
        for i, L in enumerate(c.lens):
            n = int(qs[i + 1] - qs[i])
            K = [[[f(x) for x in r] for r in tok] for tok in c.Klog[i]]
            V = [[[f(x) for x in r] for r in tok] for tok in c.Vlog[i]]
            for j in range(n):
                p = L - n + j
                qq = [[f(x) for x in row] for row in q[qs[i] + j]]
                want = np.array(brute_force(qq, K[:p + 1], V[:p + 1], c.scale))
                assert np.max(np.abs(got[qs[i] + j] - want)) <= 1e-12, (dtype, i, j)


def pin_prefill_closed_forms(o):
    """The pages' 6-token prompt ([explain] Step 6): the first token sees only itself, so its output is
    its own V row exactly; with q = 0 every row is the running mean of V."""
    rng = np.random.default_rng(26)
    c, q, qs = _prefill_case(rng, [6], [6], H=3, D=16)
    out = o.prefill(q, c.k_pool, c.v_pool, c.tables, qs, c.context_lens, 0.7, c.bs, "f32")
    assert np.array_equal(out[0], c.Vlog[0][0].astype(np.float64))
    q[:] = 0
    out = o.prefill(q, c.k_pool, c.v_pool, c.tables, qs, c.context_lens, 0.7, c.bs, "f32")
    for j in range(6):
        assert np.max(np.abs(out[j] - c.Vlog[0][:j + 1].astype(np.float64).mean(axis=0))) <= 1e-12


def pin_prefill_causality(o):
    """Changing a token's K/V changes the rows at or after its position and none before."""
    rng = np.random.default_rng(27)
    c, q, qs = _prefill_case(rng, [40], [40])
    base = o.prefill(q, c.k_pool, c.v_pool, c.tables, qs, c.context_lens, c.scale, c.bs, "f32")
    t = 23
    b, off = c.tables[0][t // c.bs], t % c.bs
    c.k_pool[b, :, off, :] += 1.0
    c.v_pool[b, :, off, :] -= 2.0
    moved = o.prefill(q, c.k_pool, c.v_pool, c.tables, qs, c.context_lens, c.scale, c.bs, "f32")
    assert np.array_equal(moved[:t], base[:t])
    assert np.all(np.max(np.abs(moved[t:] - base[t:]), axis=(1, 2)) > 0)


def pin_prefill_prefix_chunks(o):
    """A chunk of new tokens after a cached prefix ([explain] Step 9) gives the same rows as the
    corresponding rows of one prefill over the whole prompt."""
    rng = np.random.default_rng(28)
    c, q, qs = _prefill_case(rng, [50, 33], [50, 33])
    full = o.prefill(q, c.k_pool, c.v_pool, c.tables, qs, c.context_lens, c.scale, c.bs, "f32")
    sel = np.concatenate([np.arange(50 - 14, 50), [50 + 32]])
    part = o.prefill(q[sel], c.k_pool, c.v_pool, c.tables, np.array([0, 14, 15]), c.context_lens, c.scale,
                     c.bs, "f32")
    assert np.max(np.abs(part - full[sel])) <= 1e-12
    # the last row of a prefill is the decode of that sequence
    dec = o.decode(q[[49, 82]], c.k_pool, c.v_pool, c.tables, c.context_lens, c.scale, c.bs, "f32")
    assert np.max(np.abs(dec - full[[49, 82]])) <= 1e-12


PINS = [pin_block_counts, pin_storage_upcast, pin_slot_example,
        pin_write_then_read, pin_write_bitwise, pin_brute_force, pin_pages_tables,
        pin_permutation_invariance, pin_poison_invariance, pin_closed_forms,
        pin_split_equals_single, pin_prefix_sharing, pin_newest_token_slots, pin_prefill_brute_force,
        pin_prefill_closed_forms, pin_prefill_causality, pin_prefill_prefix_chunks]


# ---------------------------------------------------------------- block pool pins
# Each takes the block-pool module (oracle.block_manager) and the oracle module.

def _front(first, num_blocks, rest_seed=0):
    """A free order that starts with ``first`` (a list) and continues with the other ids shuffled."""
    rest = [b for b in np.random.default_rng(rest_seed).permutation(num_blocks).tolist() if b not in first]
    return list(first) + rest


def pin_pool_block42_flow(bm, o):
    g = golden("block_pool.json")["block42"]
    bs = g["block_size"]
    pool = bm.BlockPool(64, bs, _front([g["first_free"], 7], 64))
    assert pool.allocate("req", g["prompt_tokens"]) == g["table_after_prefill"]
    slots, copies = pool.append_slots("req", 1)
    assert slots == [g["first_decode_slot"]] and copies == []
    slots, _ = pool.append_slots("req", g["block_full_after_tokens"] - g["prompt_tokens"] - 1)
    assert slots == list(range(42 * bs + 7, 42 * bs + bs)) and pool.table("req") == [42]
    slots, copies = pool.append_slots("req", 1)                  # token 16: a new block
    assert pool.table("req") == [42, 7] and slots == [7 * bs] and copies == []
    free_before = pool.num_free()
    assert pool.free_sequence("req") == [42, 7] and pool.num_free() == free_before + 2
    assert pool.allocate("next", 20) == [42, 7]                   # immediately reused


def pin_pool_prefix_full_block(bm, o):
    g = golden("block_pool.json")["prefix_sharing"]
    bs, shared = g["block_size"], g["shared_block"]
    own = g["own_blocks"]
    pool = bm.BlockPool(100, bs, _front([shared, own["A"], own["B"], own["C"]], 100))
    pool.allocate("prompt", bs)                                   # a prefix that fills block 5
    for r in ("A", "B", "C"):
        pool.fork("prompt", r)
    pool.free_sequence("prompt")
    assert pool.refcount[shared] == g["refcount"]
    for r in ("A", "B", "C"):
        slots, copies = pool.append_slots(r, 1)
        assert copies == [] and slots == [own[r] * bs]
        assert pool.table(r) == [shared, own[r]]
    assert pool.refcount[shared] == 3


def pin_pool_copy_on_write(bm, o):
    g = golden("block_pool.json")["prefix_sharing"]
    bs, shared, n = g["block_size"], g["shared_block"], g["short_prompt_tokens"]
    pool = bm.BlockPool(100, bs, _front([shared, 40, 41, 42], 100))
    pool.allocate("prompt", n)
    for r in ("A", "B", "C"):
        pool.fork("prompt", r)
    assert pool.refcount[shared] == 4
    slots, copies = pool.append_slots("A", 1)                    # write into the shared block: copy
    assert copies == [(shared, 40)] and slots == [40 * bs + n]
    assert pool.table("A") == [40] and pool.table("B") == [shared] and pool.refcount[shared] == 3
    slots, copies = pool.append_slots("A", 2)                    # A's block is private now
    assert copies == [] and slots == [40 * bs + n + 1, 40 * bs + n + 2]
    assert pool.append_slots("B", 1)[1] == [(shared, 41)]
    assert pool.append_slots("C", 1)[1] == [(shared, 42)]
    assert pool.refcount[shared] == 1 and pool.table("prompt") == [shared]
    # once only one table holds it, its owner writes in place
    assert pool.append_slots("prompt", 1) == ([shared * bs + n], [])


def pin_pool_parallel_sampling(bm, o):
    g = golden("block_pool.json")["parallel_sampling"]
    bs, L, n = g["block_size"], g["prompt_tokens"], g["samples"]
    pool = bm.BlockPool(64, bs)
    pool.allocate(0, L)
    for s in range(1, n):
        pool.fork(0, s)
    copies = []
    for s in range(n):
        copies += pool.append_slots(s, 1)[1]
    in_use = 64 - pool.num_free()
    assert in_use == g["blocks_shared_after_one_token"] and len(copies) == n - 1
    assert n * -(-(L + 1) // bs) == g["blocks_unshared"]
    full = pool.table(0)[:L // bs]
    assert all(pool.table(s)[:L // bs] == full for s in range(n))          # full prompt blocks stay shared
    assert len({pool.table(s)[-1] for s in range(n)}) == n                  # each sample owns its last block


def _check_pool_invariants(pool):
    count = [0] * pool.num_blocks
    for seq, t in pool.tables.items():
        assert len(t) == -(-pool.tokens[seq] // pool.block_size), seq
        for b in t:
            count[b] += 1
    assert count == pool.refcount
    free = set(pool.free)
    assert len(free) == len(pool.free)
    assert all((count[b] == 0) == (b in free) for b in range(pool.num_blocks))


def _random_ops(bm, rng, pool, steps, on=None):
    """Random allocate / fork / append / free on ``pool``; ``on`` maps event names to callbacks."""
    on = on or {}
    live, next_id = [], 0

    def event(name, *args):
        if name in on:
            on[name](*args)

    for _ in range(steps):
        r = rng.random()
        try:
            if r < 0.25 or not live:
                pool.allocate(next_id, int(rng.integers(1, 60)))
                event("allocate", next_id)
                live.append(next_id)
                next_id += 1
            elif r < 0.4:
                parent = live[int(rng.integers(len(live)))]
                pool.fork(parent, next_id)
                event("fork", parent, next_id)
                live.append(next_id)
                next_id += 1
            elif r < 0.85:
                s = live[int(rng.integers(len(live)))]
                slots, copies = pool.append_slots(s, int(rng.integers(1, 20)))
                event("append", s, slots, copies)
            else:
                s = live.pop(int(rng.integers(len(live))))
                pool.free_sequence(s)
                event("free", s)
        except bm.OutOfBlocks:
            if live:
                s = live.pop(0)
                pool.free_sequence(s)
                event("free", s)
        _check_pool_invariants(pool)
        yield live


def pin_pool_invariants(bm, o):
    rng = np.random.default_rng(21)
    pool = bm.BlockPool(48, 16, rng.permutation(48))
    for live in _random_ops(bm, rng, pool, 400):
        for s in live:                          # every token's slot index falls inside the table
            assert pool.tokens[s] <= len(pool.table(s)) * pool.block_size


def pin_pool_contents(bm, o):
    """Data-level check: sequences keep exactly their own tokens through shared prefixes,
    copy-on-write, appends and frees (copies via copy_blocks, writes via the oracle's kv_write)."""
    rng = np.random.default_rng(22)
    NB, H, bs, D = 40, 2, 8, 4
    pool = bm.BlockPool(NB, bs, rng.permutation(NB))
    st = {"k": np.full((NB, H, bs, D), np.nan, dtype=np.float32),
          "v": np.full((NB, H, bs, D), np.nan, dtype=np.float32)}
    expect = {}

    def write(seq, slots):
        kn = rng.standard_normal((len(slots), H, D)).astype(np.float32)
        vn = rng.standard_normal((len(slots), H, D)).astype(np.float32)
        st["k"], st["v"] = o.kv_write(kn, vn, np.array(slots), st["k"], st["v"], bs)
        old_k, old_v = expect.get(seq, (np.zeros((0, H, D), np.float32), np.zeros((0, H, D), np.float32)))
        expect[seq] = (np.concatenate([old_k, kn]), np.concatenate([old_v, vn]))

    def on_allocate(seq):
        t = pool.table(seq)
        write(seq, [t[i // bs] * bs + i % bs for i in range(pool.tokens[seq])])

    def on_append(seq, slots, copies):
        st["k"], st["v"] = bm.copy_blocks(st["k"], st["v"], copies)
        write(seq, slots)

    on = {"allocate": on_allocate, "append": on_append,
          "fork": lambda p, c: expect.__setitem__(c, expect[p]), "free": lambda s: expect.pop(s)}
    for live in _random_ops(bm, rng, pool, 300, on):
        for s in live:
            t, L = pool.table(s), pool.tokens[s]
            K = o.gather_sequence(st["k"], t, L, bs, "f32")
            V = o.gather_sequence(st["v"], t, L, bs, "f32")
            assert np.array_equal(K, expect[s][0].transpose(1, 0, 2)), s
            assert np.array_equal(V, expect[s][1].transpose(1, 0, 2)), s


def pin_copy_blocks(bm, o):
    rng = np.random.default_rng(23)
    NB, H, bs, D = 12, 3, 16, 8
    k = rng.standard_normal((NB, H, bs, D)).astype(np.float32)
    v = rng.standard_normal((NB, H, bs, D)).astype(np.float32)
    k[2, 1, 5, 3] = np.float32(np.nan)
    k[2, 0, 0, 0] = np.float32(-0.0)
    pairs = [(2, 9), (4, 0), (2, 11)]
    k2, v2 = bm.copy_blocks(k, v, pairs)
    for s, d in pairs:
        assert np.array_equal(k2[d].view(np.uint32), k[s].view(np.uint32))
        assert np.array_equal(v2[d].view(np.uint32), v[s].view(np.uint32))
    untouched = [b for b in range(NB) if b not in (9, 0, 11)]
    assert np.array_equal(k2[untouched].view(np.uint32), k[untouched].view(np.uint32))
    assert np.array_equal(v2[untouched].view(np.uint32), v[untouched].view(np.uint32))


def pin_pool_waste_example(bm, o):
    """The pages' A100 / LLaMA-2-13B comparison: static reservation vs 16-token blocks."""
    g = golden("waste.json")
    bs, mb = g["block_size"], g["mb_per_token"]
    pool = bm.BlockPool(100, bs)
    for i, L in enumerate(g["lens"]):
        pool.allocate(i, L)
    u = bm.usage(pool)
    assert u["used_blocks"] == g["paged_blocks"] and u["stored_tokens"] == g["used_tokens"]
    assert u["logical_tokens"] == g["used_tokens"] and u["sequences"] == len(g["lens"])
    assert u["allocated_slots"] - u["stored_tokens"] == g["empty_slots"]
    assert [len(pool.table(i)) * bs - L for i, L in enumerate(g["lens"])] == g["empty_slots_per_request"]
    assert abs(bm.paged_waste(u) - g["paged_waste"]) < 1e-12
    static = u["sequences"] * g["max_model_len"]
    assert static == g["static_slots"]
    assert abs(static * mb - g["static_mb_approx"]) / g["static_mb_approx"] < 0.01
    assert abs(u["stored_tokens"] * mb - g["used_mb_approx"]) < 1.0
    assert abs(u["allocated_slots"] * mb - g["paged_mb_approx"]) < 1.0
    assert round(bm.static_waste(u, g["max_model_len"]), 2) == g["static_waste_approx"]
    for L, empty in g["why_below_4_percent"]["cases"]:
        p = bm.BlockPool(8, bs)
        p.allocate(0, L)
        uu = bm.usage(p)
        assert uu["allocated_slots"] - uu["stored_tokens"] == empty
    # sharing: a forked prompt's blocks are stored once but read by both sequences
    p = bm.BlockPool(16, bs)
    p.allocate(0, 40)
    p.fork(0, 1)
    uu = bm.usage(p)
    assert uu["stored_tokens"] == 40 and uu["logical_tokens"] == 80 and uu["shared_blocks"] == 3
    assert abs(bm.paged_waste(uu) - 8 / 48) < 1e-12            # the third block's 8 empty slots
    p.append_slots(1, 1)                       # copy-on-write of the partly filled third block
    uu = bm.usage(p)
    assert uu["stored_tokens"] == 16 + 16 + 8 + 9 and uu["used_blocks"] == 4 and uu["shared_blocks"] == 2


POOL_PINS = [pin_pool_block42_flow, pin_pool_prefix_full_block, pin_pool_copy_on_write,
             pin_pool_parallel_sampling, pin_pool_invariants, pin_pool_contents, pin_copy_blocks,
             pin_pool_waste_example]
