"""GPU parity of the continuous-batching decode loop: many steps of admissions, forks (parallel
samples), appends with copy-on-write, and releases at each request's end, with the library's block pool,
batch planner and kernels (DecodeLoop) against the oracle's block pool, copy, write, slot rule and
attention, step by step.

Bars: block tables, context lengths and slot mappings on the device equal the oracle's exactly; the
caches are bit-exact; attention is within max-abs 1e-5 (fp32) or max-abs 2e-2 and relative L2 5e-3
(bf16) of the float64 oracle.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import oracle.block_manager as BM
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_383_amd import build as b
    b.ensure_built()
    import paged_kv_cache_383_amd as m
    m.lib()
    return m


def storage(rng, shape, dt):
    x = rng.standard_normal(shape).astype(np.float32)
    if dt == "f32":
        return x
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def dev(a, dt):
    a = np.ascontiguousarray(a)
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view({2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


@pytest.mark.parametrize("dt,D", [("f32", 64), ("bf16", 128)])
def test_decode_loop_matches_oracle(pkv, dt, D):
    from paged_kv_cache_383_amd.decode_loop import DecodeLoop
    rng = np.random.default_rng(400 + D)
    rows, H, bs, NB, width = 5, 3, 16, 110, 20
    order = rng.permutation(NB)
    nan = np.float32(np.nan) if dt == "f32" else np.uint16(0x7FC0)
    k_ref = np.full((NB, H, bs, D), nan, dtype=np.float32 if dt == "f32" else np.uint16)
    v_ref = k_ref.copy()
    loop = DecodeLoop(dev(k_ref, dt), dev(v_ref, dt), rows, width, free_order=order)
    ref = BM.BlockPool(NB, bs, order)
    # requests: (prompt length, tokens to generate, index of the request it samples from or None)
    reqs = []
    for i in range(16):
        fork_of = i - 1 if i % 4 == 3 else None
        reqs.append((int(rng.integers(1, 120)), int(rng.integers(1, 45)), fork_of))
    row_req, gen = [-1] * rows, [0] * rows
    seq_of = {}
    nxt, done, steps = 0, 0, 0
    scale = loop.scale
    while done < len(reqs):
        for r in range(rows):                              # fill idle rows, in row order
            if row_req[r] >= 0 or nxt >= len(reqs):
                continue
            P, G, fork_of = reqs[nxt]
            parent = seq_of.get(fork_of) if fork_of is not None else None
            if parent is not None and parent in ref.tables:
                loop.fork(r, parent, nxt)
                ref.fork(parent, nxt)
            else:
                kp, vp = storage(rng, (P, H, D), dt), storage(rng, (P, H, D), dt)
                loop.admit(r, nxt, dev(kp, dt), dev(vp, dt))
                t = ref.allocate(nxt, P)
                sl = np.array([t[i // bs] * bs + i % bs for i in range(P)])
                k_ref, v_ref = oracle.kv_write(kp, vp, sl, k_ref, v_ref, bs)
            seq_of[nxt] = nxt
            row_req[r], gen[r] = nxt, 0
            nxt += 1
        q = storage(rng, (rows, H, D), dt)
        kn, vn = storage(rng, (rows, H, D), dt), storage(rng, (rows, H, D), dt)
        out = loop.step(dev(q, dt), dev(kn, dt), dev(vn, dt))
        slots, copies = np.full(rows, -1, dtype=np.int64), []
        for r in range(rows):
            if row_req[r] >= 0:
                s, c = ref.append_slots(row_req[r], 1)
                slots[r] = s[0]
                copies += c
        k_ref, v_ref = BM.copy_blocks(k_ref, v_ref, copies)
        k_ref, v_ref = oracle.kv_write(kn, vn, slots, k_ref, v_ref, bs)
        tables = np.full((rows, width), -1, dtype=np.int32)
        lens = np.zeros(rows, dtype=np.int32)
        for r in range(rows):
            if row_req[r] >= 0:
                t = ref.table(row_req[r])
                tables[r, :len(t)] = t
                lens[r] = ref.tokens[row_req[r]]
        torch.cuda.synchronize()
        assert np.array_equal(loop.tables.cpu().numpy(), tables), steps
        assert np.array_equal(loop.lens.cpu().numpy(), lens), steps
        assert np.array_equal(loop.slots.cpu().numpy(), slots), steps
        assert np.array_equal(oracle.newest_token_slots(tables, lens, bs), slots)
        want = oracle.decode(q, k_ref, v_ref, tables, lens, scale, bs, dt)
        got = out.double().cpu().numpy()
        err = float(np.max(np.abs(got - want)))
        if dt == "f32":
            assert err <= 1e-5, (steps, err)
        else:
            live = lens > 0
            rel = np.linalg.norm(got[live] - want[live]) / np.linalg.norm(want[live])
            assert err <= 2e-2 and rel <= 5e-3, (steps, err, rel)
        if steps % 10 == 0:
            assert np.array_equal(bits(W.storage_numpy(loop.k_cache)), bits(k_ref))
            assert np.array_equal(bits(W.storage_numpy(loop.v_cache)), bits(v_ref))
        for r in range(rows):                              # requests that reached their length end
            if row_req[r] >= 0:
                gen[r] += 1
                if gen[r] == reqs[row_req[r]][1]:
                    loop.release(r)
                    ref.free_sequence(row_req[r])
                    row_req[r] = -1
                    done += 1
        steps += 1
        if steps % 20 == 0:
            print(f"[loop] {dt} D={D}: step {steps}, {done} of {len(reqs)} requests done", flush=True)
    assert loop.pool.num_free() == NB and ref.num_free() == NB     # every block came back
    print(f"[loop] {dt} D={D}: {steps} steps", flush=True)
