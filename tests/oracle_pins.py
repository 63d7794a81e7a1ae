"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load(path)``)
and raises ``AssertionError`` (or ``oracle.OracleError``) when the oracle is
wrong. ``test_oracle.py`` runs them against the real oracle, and
``test_oracle_mutants.py`` runs them against copies of the oracle with one
planted mistake each, expecting at least one pin to fail for every mistake.

Kinds of pin used (none retypes the oracle's own loops):
  * a library routine: torch's scaled_dot_product_attention in fp64 on a
    contiguous cache that the test lays out itself;
  * brute force: a scalar Python loop with math.fsum and no max shift;
  * closed forms: two-token softmax, uniform keys, zero scale, constant V,
    one-hot V, the large-logit limit, a single token;
  * invariants from the pages: placement of blocks anywhere in the pool does
    not change the result ("Why this wins", Idea 1 of the day-9 post), and
    requests that share prefix blocks read the same values as unshared copies
    (same section, "Sharing");
  * the cache write, checked position by position with numpy indexing.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

B = 16


# --------------------------------------------------------------------------
# Test-side layout helpers (numpy slicing; independent of the oracle's loops)
# --------------------------------------------------------------------------

def paged_from_contiguous(Ks, Vs, rng, block_size=B, extra_blocks=3, pad=-1, poison=True):
    """Place per-sequence contiguous K/V ([L, Hkv, D] each) into randomly permuted
    physical blocks. Returns (key_cache, value_cache, block_tables)."""
    Hkv, D = Ks[0].shape[1], Ks[0].shape[2]
    nblk = [-(-k.shape[0] // block_size) for k in Ks]
    NB = sum(nblk) + extra_blocks
    fill = np.nan if poison else 0.0
    kc = np.full((NB, Hkv, block_size, D), fill)
    vc = np.full((NB, Hkv, block_size, D), fill)
    MB = max(max(nblk), 1)
    tables = np.full((len(Ks), MB), pad, dtype=np.int32)
    perm = rng.permutation(NB)
    cur = 0
    for s, (k, v) in enumerate(zip(Ks, Vs)):
        for j in range(nblk[s]):
            b = int(perm[cur])
            cur += 1
            tables[s, j] = b
            rows_k = k[j * block_size:(j + 1) * block_size]        # [n, Hkv, D]
            rows_v = v[j * block_size:(j + 1) * block_size]
            kc[b, :, :rows_k.shape[0], :] = rows_k.transpose(1, 0, 2)
            vc[b, :, :rows_v.shape[0], :] = rows_v.transpose(1, 0, 2)
    if pad == -2:   # point padding at a NaN-filled spare block
        spare = int(perm[cur])
        for s in range(len(Ks)):
            tables[s, nblk[s]:] = spare
    return kc, vc, tables


def random_problem(rng, lengths, Hq, Hkv, D, scale=None, pad=-1, poison=True):
    Ks = [rng.standard_normal((L, Hkv, D)) for L in lengths]
    Vs = [rng.standard_normal((L, Hkv, D)) for L in lengths]
    q = rng.standard_normal((len(lengths), Hq, D))
    kc, vc, bt = paged_from_contiguous(Ks, Vs, rng, pad=pad, poison=poison)
    cl = np.asarray(lengths, dtype=np.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return dict(q=q, Ks=Ks, Vs=Vs, kc=kc, vc=vc, bt=bt, cl=cl, scale=scale)


def run(lib, p, **kw):
    return oracle.decode(p["q"], p["kc"], p["vc"], p["bt"], p["cl"], p["scale"], lib=lib, **kw)


# --------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------

def pin_sdpa_library(lib):
    """Oracle == torch SDPA (fp64, CPU) on the contiguous cache, GQA by repeat_interleave."""
    rng = np.random.default_rng(11)
    lengths = [1, 5, 16, 17, 40, 64]
    Hq, Hkv, D = 8, 2, 24
    p = random_problem(rng, lengths, Hq, Hkv, D, scale=0.3)
    out = run(lib, p)
    sc = oracle.fp32_scale(p["scale"])
    for s, L in enumerate(lengths):
        q = torch.from_numpy(p["q"][s]).reshape(1, Hq, 1, D)
        k = torch.from_numpy(p["Ks"][s]).permute(1, 0, 2).reshape(1, Hkv, L, D)
        v = torch.from_numpy(p["Vs"][s]).permute(1, 0, 2).reshape(1, Hkv, L, D)
        k = k.repeat_interleave(Hq // Hkv, dim=1).contiguous()
        v = v.repeat_interleave(Hq // Hkv, dim=1).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=sc)
        np.testing.assert_allclose(out[s], ref.reshape(Hq, D).numpy(), rtol=0, atol=1e-12)


def pin_brute_force(lib):
    """A scalar Python loop (no max shift, math.fsum) on tiny inputs agrees to 1e-12."""
    rng = np.random.default_rng(12)
    lengths = [1, 3, 20, 33]
    Hq, Hkv, D = 4, 2, 5
    p = random_problem(rng, lengths, Hq, Hkv, D, scale=0.5)
    out = run(lib, p)
    sc = oracle.fp32_scale(p["scale"])
    G = Hq // Hkv
    for s, L in enumerate(lengths):
        for h in range(Hq):
            kv = h // G
            e = []
            for t in range(L):
                blk, off = divmod(t, B)
                b = p["bt"][s][blk]
                kvec = p["kc"][b][kv][off]
                e.append(math.exp(sc * math.fsum(p["q"][s][h][d] * kvec[d] for d in range(D))))
            z = math.fsum(e)
            for d in range(D):
                ref = math.fsum(e[t] / z * p["vc"][p["bt"][s][t // B]][kv][t % B][d]
                                for t in range(L))
                assert abs(out[s][h][d] - ref) < 1e-12, (s, h, d, out[s][h][d], ref)


def pin_single_token(lib):
    """A context of one token returns that token's V exactly (w = 1)."""
    rng = np.random.default_rng(13)
    p = random_problem(rng, [1, 1, 1], Hq=6, Hkv=3, D=8)
    out = run(lib, p)
    for s in range(3):
        for h in range(6):
            assert np.array_equal(out[s, h], p["Vs"][s][0, h // 2]), (s, h)


def pin_constant_values(lib):
    """V == 1 everywhere gives out == 1 (the weights sum to one)."""
    rng = np.random.default_rng(14)
    p = random_problem(rng, [7, 16, 29, 50], Hq=4, Hkv=4, D=8)
    live = ~np.isnan(p["vc"])
    p["vc"][live] = 1.0
    out = run(lib, p)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)


def pin_gqa_head_map(lib):
    """With V of KV head k constant k + 1, query head h returns h // G + 1."""
    rng = np.random.default_rng(15)
    Hq, Hkv = 12, 3
    p = random_problem(rng, [5, 18, 31], Hq=Hq, Hkv=Hkv, D=4)
    for k in range(Hkv):
        sl = p["vc"][:, k]
        sl[~np.isnan(sl)] = k + 1.0
    out = run(lib, p)
    for h in range(Hq):
        np.testing.assert_allclose(out[:, h], h // (Hq // Hkv) + 1.0, rtol=0, atol=1e-13)


def pin_two_token_closed_form(lib):
    """Two tokens with logits 0 and +/-ln 3 have weights (1/4, 3/4) or (3/4, 1/4)."""
    D = 2
    for sign, expect in ((1.0, (1.0, 3.0)), (-1.0, (3.0, 1.0))):
        scale = 0.125                                   # exact in fp32
        a = sign * 8.0 * math.log(3.0)                  # scale * a = +/- ln 3
        q = np.array([[[a, 0.0]]])
        K = [np.array([[[0.0, 0.0]], [[1.0, 0.0]]])]    # [L=2, Hkv=1, D]
        V = [np.array([[[4.0, 0.0]], [[0.0, 4.0]]])]
        kc, vc, bt = paged_from_contiguous(K, V, np.random.default_rng(16))
        out = oracle.decode(q, kc, vc, bt, np.array([2], np.int32), scale, lib=lib)
        np.testing.assert_allclose(out[0, 0], expect, rtol=0, atol=1e-13)


def pin_uniform_keys(lib):
    """All keys equal gives uniform weights: out is the mean of V."""
    rng = np.random.default_rng(17)
    lengths = [3, 16, 37]
    p = random_problem(rng, lengths, Hq=2, Hkv=1, D=6)
    for s in range(len(lengths)):
        p["Ks"][s][:] = p["Ks"][s][0]
    kc, vc, bt = paged_from_contiguous(p["Ks"], p["Vs"], rng)
    out = oracle.decode(p["q"], kc, vc, bt, p["cl"], 0.7, lib=lib)
    for s in range(len(lengths)):
        np.testing.assert_allclose(out[s], np.broadcast_to(p["Vs"][s][:, 0].mean(0), (2, 6)),
                                   rtol=0, atol=1e-13)


def pin_zero_scale(lib):
    """scale = 0 makes every logit 0: out is the mean of V."""
    rng = np.random.default_rng(18)
    lengths = [2, 17, 40]
    p = random_problem(rng, lengths, Hq=3, Hkv=3, D=5, scale=0.0)
    out = run(lib, p)
    for s in range(len(lengths)):
        np.testing.assert_allclose(out[s], p["Vs"][s].mean(0), rtol=0, atol=1e-13)


def pin_large_logits(lib):
    """Huge logits do not overflow; the output is the V of the top-scoring token,
    including when that token is the first one."""
    rng = np.random.default_rng(19)
    D = 4
    for top in (0, 9, 22):
        L = 23
        K = rng.standard_normal((L, 1, D)) * 0.1
        K[top, 0] = np.array([1.0, 0.0, 0.0, 0.0])
        V = [rng.standard_normal((L, 1, D))]
        q = np.array([[[1e6, 0.0, 0.0, 0.0]]])
        kc, vc, bt = paged_from_contiguous([K], V, rng)
        out = oracle.decode(q, kc, vc, bt, np.array([L], np.int32), 1.0, lib=lib)
        assert np.all(np.isfinite(out))
        np.testing.assert_allclose(out[0, 0], V[0][top, 0], rtol=0, atol=1e-12)


def pin_one_hot_weights(lib):
    """With V_t = e_t (L <= D), out[h][t] is the weight of token t: non-negative, sums to
    one, and w_t / w_u = exp(l_t - l_u) with logits from numpy."""
    rng = np.random.default_rng(20)
    L, D, Hq = 19, 24, 2
    K = rng.standard_normal((L, 1, D))
    V = np.zeros((L, 1, D))
    V[np.arange(L), 0, np.arange(L)] = 1.0
    q = rng.standard_normal((1, Hq, D))
    scale = 0.25
    kc, vc, bt = paged_from_contiguous([K], [V], rng)
    out = oracle.decode(q, kc, vc, bt, np.array([L], np.int32), scale, lib=lib)
    for h in range(Hq):
        w = out[0, h, :L]
        assert np.all(w >= 0) and np.all(out[0, h, L:] == 0)
        assert abs(w.sum() - 1.0) < 1e-14
        logits = scale * (K[:, 0, :] @ q[0, h])
        np.testing.assert_allclose(np.log(w / w[0]), logits - logits[0], rtol=0, atol=1e-11)


def pin_block_permutation(lib):
    """Moving blocks elsewhere in the pool (and fixing the tables) changes nothing, bit for bit."""
    rng = np.random.default_rng(21)
    p = random_problem(rng, [4, 16, 45, 63], Hq=4, Hkv=2, D=8)
    base = run(lib, p)
    NB = p["kc"].shape[0]
    perm = rng.permutation(NB)                  # new home of each physical block
    kc2 = np.empty_like(p["kc"])
    vc2 = np.empty_like(p["vc"])
    kc2[perm] = p["kc"]
    vc2[perm] = p["vc"]
    bt2 = np.where(p["bt"] >= 0, perm[np.maximum(p["bt"], 0)], -1).astype(np.int32)
    out2 = oracle.decode(p["q"], kc2, vc2, bt2, p["cl"], p["scale"], lib=lib)
    assert np.array_equal(base, out2)


def pin_prefix_sharing(lib):
    """Sequences that share prefix blocks give the same result as with private copies."""
    rng = np.random.default_rng(22)
    Hkv, D, Hq = 2, 8, 4
    prefix = [rng.standard_normal((32, Hkv, D)), rng.standard_normal((32, Hkv, D))]
    pk, pv = prefix
    suffix = [7, 16, 20]
    Ks = [np.concatenate([pk, rng.standard_normal((n, Hkv, D))]) for n in suffix]
    Vs = [np.concatenate([pv, rng.standard_normal((n, Hkv, D))]) for n in suffix]
    q = rng.standard_normal((3, Hq, D))
    kc, vc, bt = paged_from_contiguous(Ks, Vs, rng)             # private copies
    cl = np.array([32 + n for n in suffix], np.int32)
    private = oracle.decode(q, kc, vc, bt, cl, 0.35, lib=lib)
    bt_shared = bt.copy()
    bt_shared[1:, :2] = bt[0, :2]                               # everyone reads seq 0's prefix
    for s in (1, 2):                                            # the abandoned copies become NaN
        kc[bt[s, :2]] = np.nan
        vc[bt[s, :2]] = np.nan
    shared = oracle.decode(q, kc, vc, bt_shared, cl, 0.35, lib=lib)
    assert np.array_equal(private, shared)


def pin_partitioned_equals_single(lib):
    """The split-context form equals the single pass (1e-12), for several partition sizes,
    and with one partition its statistics are the single pass's."""
    rng = np.random.default_rng(23)
    lengths = [1, 15, 16, 17, 64, 100]
    p = random_problem(rng, lengths, Hq=4, Hkv=2, D=8)
    single = run(lib, p)
    for P in (16, 32, 48, 128):
        out, pm, ps, po = oracle.decode_partitioned(p["q"], p["kc"], p["vc"], p["bt"], p["cl"],
                                                    p["scale"], P, lib=lib)
        np.testing.assert_allclose(out, single, rtol=0, atol=1e-12)
    out, pm, ps, po = oracle.decode_partitioned(p["q"], p["kc"], p["vc"], p["bt"], p["cl"],
                                                p["scale"], 128, lib=lib)
    np.testing.assert_allclose(po[:, :, 0, :], single, rtol=0, atol=1e-14)


def pin_partition_stats(lib):
    """Per-partition max and sum against logits computed by numpy, and empty partitions."""
    rng = np.random.default_rng(24)
    lengths = [40, 7]
    Hq, Hkv, D, P = 2, 1, 6, 16
    p = random_problem(rng, lengths, Hq=Hq, Hkv=Hkv, D=D)
    sc = oracle.fp32_scale(p["scale"])
    out, pm, ps, po = oracle.decode_partitioned(p["q"], p["kc"], p["vc"], p["bt"], p["cl"],
                                                p["scale"], P, lib=lib)
    for s, L in enumerate(lengths):
        for h in range(Hq):
            logits = sc * (p["Ks"][s][:, 0, :] @ p["q"][s, h])
            for part in range(pm.shape[2]):
                seg = logits[part * P:min((part + 1) * P, L)]
                if len(seg) == 0:
                    assert pm[s, h, part] == -np.inf and ps[s, h, part] == 0
                    assert np.all(po[s, h, part] == 0)
                    continue
                assert abs(pm[s, h, part] - seg.max()) < 1e-13
                assert abs(ps[s, h, part] - np.exp(seg - seg.max()).sum()) < 1e-12


def pin_zero_length(lib):
    """A context of length 0 gives a zero row; other rows are unaffected."""
    rng = np.random.default_rng(25)
    p = random_problem(rng, [0, 9], Hq=2, Hkv=1, D=4)
    out = run(lib, p)
    assert np.all(out[0] == 0)
    out2, *_ = oracle.decode_partitioned(p["q"], p["kc"], p["vc"], p["bt"], p["cl"], p["scale"],
                                         16, lib=lib)
    assert np.all(out2[0] == 0)
    np.testing.assert_allclose(out2[1], out[1], rtol=0, atol=1e-13)


def pin_poison_not_read(lib):
    """NaN in unused blocks, block tails and a padding block never reaches the output."""
    rng = np.random.default_rng(26)
    p = random_problem(rng, [3, 16, 18, 47], Hq=4, Hkv=2, D=8, pad=-2)
    out = run(lib, p)
    assert np.all(np.isfinite(out))
    out2, *_ = oracle.decode_partitioned(p["q"], p["kc"], p["vc"], p["bt"], p["cl"], p["scale"],
                                         32, lib=lib)
    assert np.all(np.isfinite(out2))


def pin_bad_tables_rejected(lib):
    """Out-of-pool block ids inside the context and over-long contexts are errors."""
    rng = np.random.default_rng(27)
    p = random_problem(rng, [20], Hq=1, Hkv=1, D=4)
    bad = p["bt"].copy()
    bad[0, 1] = p["kc"].shape[0]
    for tables, lens in ((bad, p["cl"]), (p["bt"], np.array([40], np.int32))):
        try:
            oracle.decode(p["q"], p["kc"], p["vc"], tables, lens, 1.0, lib=lib)
        except oracle.OracleError:
            continue
        raise AssertionError("invalid table accepted")


def pin_scatter_positions(lib):
    """The cache write puts token i, head h at [slot // 16, h, slot % 16], bit for bit
    (NaN payloads included), skips negative slots and touches nothing else."""
    rng = np.random.default_rng(28)
    NB, Hkv, D, T = 6, 3, 8, 7
    kc = rng.integers(0, 1 << 16, size=(NB, Hkv, B, D), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(NB, Hkv, B, D), dtype=np.uint16)
    key = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    value = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    key[0, 0, 0] = 0x7FC1          # a bf16 NaN with a payload
    slots = np.array([5, -1, 17, 95, 48, -3, 0], np.int64)
    kc0, vc0 = kc.copy(), vc.copy()
    oracle.reshape_and_cache(key, value, kc, vc, slots, lib=lib)
    ek, ev = kc0.copy(), vc0.copy()
    for i, slot in enumerate(slots):
        if slot >= 0:
            ek[slot // B, :, slot % B, :] = key[i]
            ev[slot // B, :, slot % B, :] = value[i]
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)
    # fp32 rows too
    kf = rng.standard_normal((2, 1, B, 4)).astype(np.float32)
    vf = kf.copy()
    kt = rng.standard_normal((1, 1, 4)).astype(np.float32)
    oracle.reshape_and_cache(kt, kt.copy(), kf, vf, np.array([31]), lib=lib)
    assert np.array_equal(kf[1, 0, 15], kt[0, 0]) and np.array_equal(vf[1, 0, 15], kt[0, 0])


def pin_scatter_rejects(lib):
    """Duplicate slots and slots past the pool are errors, and nothing is written."""
    rng = np.random.default_rng(29)
    kc = rng.integers(0, 1 << 16, size=(2, 1, B, 4), dtype=np.uint16)
    vc = kc.copy()
    key = rng.integers(0, 1 << 16, size=(2, 1, 4), dtype=np.uint16)
    for slots in ([3, 3], [3, 32]):
        k0 = kc.copy()
        try:
            oracle.reshape_and_cache(key, key.copy(), kc, vc, np.array(slots, np.int64), lib=lib)
        except oracle.OracleError:
            assert np.array_equal(kc, k0)
            continue
        raise AssertionError(f"slots {slots} accepted")


def pin_copy_blocks_positions(lib):
    """Copy-on-write: block dst of both pools becomes block src, bit for bit, for every
    head and row; pairs with a negative id are skipped; nothing else changes (day-9 post,
    "Why this wins": only the changed block is copied)."""
    rng = np.random.default_rng(30)
    NB, Hkv, D = 9, 3, 8
    kc = rng.integers(0, 1 << 16, size=(NB, Hkv, B, D), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(NB, Hkv, B, D), dtype=np.uint16)
    kc[2, 1, 3, 0] = 0x7FC1
    pairs = np.array([[2, 5], [-1, 0], [7, 1], [2, 8], [4, -1]], np.int64)
    ek, ev = kc.copy(), vc.copy()
    for src, dst in pairs:
        if src >= 0 and dst >= 0:
            ek[dst] = kc[src]
            ev[dst] = vc[src]
    oracle.copy_blocks(kc, vc, pairs, lib=lib)
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)
    assert np.array_equal(kc[5], kc[2]) and not np.array_equal(kc[5], vc[5])
    f = rng.standard_normal((3, 1, B, 4)).astype(np.float32)
    g = rng.standard_normal((3, 1, B, 4)).astype(np.float32)
    f0, g0 = f.copy(), g.copy()
    oracle.copy_blocks(f, g, [[0, 2]], lib=lib)
    assert np.array_equal(f[2], f0[0]) and np.array_equal(g[2], g0[0])
    assert np.array_equal(f[:2], f0[:2]) and np.array_equal(g[:2], g0[:2])


def pin_copy_blocks_rejects(lib):
    """Copies whose result would depend on their order (a repeated destination, a
    destination that is a source) and ids past the pool are errors; nothing is written."""
    rng = np.random.default_rng(31)
    kc = rng.integers(0, 1 << 16, size=(4, 1, B, 4), dtype=np.uint16)
    vc = kc.copy()
    for pairs in ([[0, 1], [2, 1]], [[0, 1], [1, 2]], [[3, 3]], [[0, 4]], [[4, 0]]):
        k0 = kc.copy()
        try:
            oracle.copy_blocks(kc, vc, pairs, lib=lib)
        except oracle.OracleError:
            assert np.array_equal(kc, k0)
            continue
        raise AssertionError(f"pairs {pairs} accepted")


def pin_swap_blocks_positions(lib):
    """Swap between two pairs of pools of different sizes: block dst of the destination
    pools becomes block src of the source pools, K from K and V from V, bit for bit (NaN
    payloads too); pairs with a negative id are skipped; the source pools and every other
    destination block are unchanged."""
    rng = np.random.default_rng(32)
    Hkv, D = 2, 8
    sk = rng.integers(0, 1 << 16, size=(7, Hkv, B, D), dtype=np.uint16)
    sv = rng.integers(0, 1 << 16, size=(7, Hkv, B, D), dtype=np.uint16)
    sk[3, 1, 15, 7] = 0x7FC3                      # a NaN payload travels as it is
    dk = rng.integers(0, 1 << 16, size=(4, Hkv, B, D), dtype=np.uint16)
    dv = rng.integers(0, 1 << 16, size=(4, Hkv, B, D), dtype=np.uint16)
    sk0, sv0, dk0, dv0 = sk.copy(), sv.copy(), dk.copy(), dv.copy()
    oracle.swap_blocks(sk, sv, dk, dv, [[3, 0], [6, 2], [-1, 1], [5, -3]], lib=lib)
    assert np.array_equal(sk, sk0) and np.array_equal(sv, sv0)
    assert np.array_equal(dk[0], sk0[3]) and np.array_equal(dv[0], sv0[3])
    assert np.array_equal(dk[2], sk0[6]) and np.array_equal(dv[2], sv0[6])
    assert np.array_equal(dk[[1, 3]], dk0[[1, 3]]) and np.array_equal(dv[[1, 3]], dv0[[1, 3]])
    assert dk[0, 1, 15, 7] == 0x7FC3


def pin_swap_round_trip_decode(lib):
    """Preemption by swapping: a sequence's blocks moved out to a second pool and back
    into different physical blocks of the first, with its table remapped, give the same
    decode output bit for bit (blocks can sit anywhere: day-9 post, "Why this wins"), and
    the blocks hold exactly their old bytes."""
    rng = np.random.default_rng(33)
    p = random_problem(rng, [37, 20], 8, 2, 16)
    ref = run(lib, p)
    kc, vc = p["kc"], p["vc"]
    NB = kc.shape[0]
    bt = p["bt"].copy()
    nblk = -(-int(p["cl"][0]) // B)
    blocks = bt[0, :nblk].astype(np.int64)
    hk = np.zeros((5,) + kc.shape[1:], kc.dtype)
    hv = np.zeros_like(hk)
    host_ids = np.array([4, 0, 2])[:nblk]
    oracle.swap_blocks(kc, vc, hk, hv, np.stack([blocks, host_ids], 1), lib=lib)
    kc2 = np.full((NB + 3,) + kc.shape[1:], np.nan, kc.dtype)
    vc2 = np.full_like(kc2, np.nan)
    kc2[:NB], vc2[:NB] = kc, vc
    kc2[blocks], vc2[blocks] = np.nan, np.nan     # the old copies are gone
    fresh = np.arange(NB, NB + nblk)
    oracle.swap_blocks(hk, hv, kc2, vc2, np.stack([host_ids, fresh], 1), lib=lib)
    bits = lambda a: a.view(np.uint64)            # tail rows hold NaN poison: compare bits
    assert np.array_equal(bits(kc2[fresh]), bits(kc[blocks]))
    assert np.array_equal(bits(vc2[fresh]), bits(vc[blocks]))
    bt[0, :nblk] = fresh
    out = run(lib, {**p, "kc": kc2, "vc": vc2, "bt": bt})
    assert np.array_equal(out, ref)


def pin_swap_blocks_rejects(lib):
    """A destination named twice, or an id past its own pool, is an error; nothing is
    written."""
    rng = np.random.default_rng(34)
    sk = rng.integers(0, 1 << 16, size=(3, 1, B, 4), dtype=np.uint16)
    dk = rng.integers(0, 1 << 16, size=(5, 1, B, 4), dtype=np.uint16)
    for pairs in ([[0, 1], [2, 1]], [[3, 0]], [[0, 5]], [[1, 2], [0, 7]]):
        d0 = dk.copy()
        try:
            oracle.swap_blocks(sk, sk.copy(), dk, dk.copy(), pairs, lib=lib)
        except oracle.OracleError:
            assert np.array_equal(dk, d0)
            continue
        raise AssertionError(f"pairs {pairs} accepted")
    oracle.swap_blocks(sk, sk.copy(), dk, dk.copy(), [[2, 4], [0, 0]], lib=lib)  # in range: fine


# --------------------------------------------------------------------------
# Multi-token queries (a prompt chunk per sequence) over the paged cache
# --------------------------------------------------------------------------

def prefill_problem(rng, lengths, nqs, Hq, Hkv, D, scale=None, poison=True):
    """random_problem plus a ragged batch of query rows: sequence s brings nqs[s] rows."""
    p = random_problem(rng, lengths, Hq, Hkv, D, scale=scale, poison=poison)
    p["qs"] = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
    p["nq"] = list(nqs)
    p["qm"] = rng.standard_normal((int(p["qs"][-1]), Hq, D))
    return p


def run_prefill(lib, p, **kw):
    return oracle.prefill(p["qm"], p["kc"], p["vc"], p["bt"], p["cl"], p["qs"], p["scale"],
                          lib=lib, **kw)


def pin_prefill_sdpa_causal(lib):
    """Multi-token queries == torch SDPA (fp64, CPU) with an explicit boolean mask: query i
    of a q-token chunk sees tokens 0 .. L - q + i of the contiguous cache."""
    rng = np.random.default_rng(31)
    lengths, nqs = [1, 7, 16, 33, 50, 40], [1, 7, 5, 16, 50, 0]
    Hq, Hkv, D = 8, 2, 24
    p = prefill_problem(rng, lengths, nqs, Hq, Hkv, D, scale=0.3)
    out = run_prefill(lib, p)
    sc = oracle.fp32_scale(p["scale"])
    for s, (L, nq) in enumerate(zip(lengths, nqs)):
        if nq == 0:
            continue
        r0 = int(p["qs"][s])
        q = torch.from_numpy(p["qm"][r0:r0 + nq]).permute(1, 0, 2).reshape(1, Hq, nq, D)
        k = torch.from_numpy(p["Ks"][s]).permute(1, 0, 2).reshape(1, Hkv, L, D)
        v = torch.from_numpy(p["Vs"][s]).permute(1, 0, 2).reshape(1, Hkv, L, D)
        k = k.repeat_interleave(Hq // Hkv, dim=1).contiguous()
        v = v.repeat_interleave(Hq // Hkv, dim=1).contiguous()
        mask = torch.arange(L)[None, :] <= (L - nq + torch.arange(nq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=sc)
        ref = ref.reshape(Hq, nq, D).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[r0:r0 + nq], ref, rtol=0, atol=1e-12)


def pin_prefill_rows_are_truncated_decodes(lib):
    """Row i of a chunk is the single-query decode of the same context cut at the row's
    position (context length L - q + i + 1), query for query."""
    rng = np.random.default_rng(32)
    lengths, nqs = [5, 20, 48, 17], [5, 3, 33, 1]
    Hq, Hkv, D = 6, 3, 16
    p = prefill_problem(rng, lengths, nqs, Hq, Hkv, D)
    out = run_prefill(lib, p)
    for s, (L, nq) in enumerate(zip(lengths, nqs)):
        r0 = int(p["qs"][s])
        for i in range(nq):
            dec = oracle.decode(p["qm"][r0 + i][None], p["kc"], p["vc"], p["bt"][s][None],
                                np.array([L - nq + i + 1], np.int32), p["scale"], lib=lib)
            np.testing.assert_allclose(out[r0 + i], dec[0], rtol=0, atol=1e-12)


def pin_prefill_brute_force(lib):
    """A scalar Python loop (no max shift, math.fsum) over the causal window, tiny inputs."""
    rng = np.random.default_rng(33)
    lengths, nqs = [3, 18, 9], [3, 4, 2]
    Hq, Hkv, D = 4, 2, 3
    p = prefill_problem(rng, lengths, nqs, Hq, Hkv, D, scale=0.7)
    out = run_prefill(lib, p)
    sc = oracle.fp32_scale(p["scale"])
    G = Hq // Hkv
    for s, (L, nq) in enumerate(zip(lengths, nqs)):
        for i in range(nq):
            row = int(p["qs"][s]) + i
            pos = L - nq + i
            for h in range(Hq):
                kv = h // G
                e = []
                for t in range(pos + 1):
                    b = p["bt"][s][t // B]
                    e.append(math.exp(sc * math.fsum(p["qm"][row][h][d] * p["kc"][b][kv][t % B][d]
                                                     for d in range(D))))
                z = math.fsum(e)
                for d in range(D):
                    ref = math.fsum(e[t] / z * p["vc"][p["bt"][s][t // B]][kv][t % B][d]
                                    for t in range(pos + 1))
                    assert abs(out[row][h][d] - ref) < 1e-12, (s, i, h, d)


def pin_prefill_first_prompt_token(lib):
    """When the chunk is the whole prompt (q = L), its first row sees token 0 alone and
    returns that token's V exactly; the others stay finite."""
    rng = np.random.default_rng(34)
    lengths = [1, 16, 37]
    Hq, Hkv, D = 4, 4, 8
    p = prefill_problem(rng, lengths, lengths, Hq, Hkv, D)
    out = run_prefill(lib, p)
    for s, L in enumerate(lengths):
        r0 = int(p["qs"][s])
        v0 = p["Vs"][s][0]                                   # [Hkv, D]
        assert np.array_equal(out[r0], v0), s
        assert np.isfinite(out[r0:r0 + L]).all()


def pin_prefill_causality(lib):
    """Changing the K and V of a context's last token changes only the row at that position
    (bit for bit: the earlier rows never read it)."""
    rng = np.random.default_rng(35)
    lengths, nqs = [30, 45], [12, 45]
    Hq, Hkv, D = 4, 2, 8
    p = prefill_problem(rng, lengths, nqs, Hq, Hkv, D)
    base = run_prefill(lib, p)
    for s, L in enumerate(lengths):
        q = dict(p)
        q["kc"], q["vc"] = p["kc"].copy(), p["vc"].copy()
        b, off = p["bt"][s][(L - 1) // B], (L - 1) % B
        q["kc"][b, :, off] += 3.0
        q["vc"][b, :, off] -= 5.0
        moved = run_prefill(lib, q)
        last = int(p["qs"][s + 1]) - 1
        changed = np.flatnonzero(np.any(moved != base, axis=(1, 2)))
        assert changed.tolist() == [last], (s, changed)


def pin_prefill_rejects(lib):
    """A chunk longer than its context, or a query_start that does not start at 0 or runs
    backwards, is an input error."""
    rng = np.random.default_rng(36)
    p = prefill_problem(rng, [5, 9], [2, 3], 2, 2, 4)
    for qs in ([0, 6, 9], [1, 3, 6], [0, 3, 2]):
        q = dict(p)
        q["qs"] = np.asarray(qs, np.int32)
        q["qm"] = np.zeros((max(qs[-1], 0), 2, 4))
        try:
            run_prefill(lib, q)
        except oracle.OracleError:
            continue
        raise AssertionError(f"query_start {qs} accepted")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
