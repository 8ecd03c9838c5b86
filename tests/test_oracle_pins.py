"""Pins of the CPU oracle against things other than itself.

The reference pages print no numeric worked example, so the oracle is pinned
by independent library routines (rocRAND's Philox, torch's fp64
scaled_dot_product_attention, scipy's logsumexp/expit), closed forms of
softmax attention, and invariants the CFR-Atlas README's "Core contract"
demands (the folded result equals full-KV attention, independent of how the
history is split into pages).  Each test names the mistake it would catch.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch
from scipy import special, stats

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


# ------------------------------------------------------------------ helpers

def _case(rng, nq, n_kv, hq, hkv, d, dtype=np.float32):
    q = rng.standard_normal((nq, hq, d)).astype(dtype)
    k = rng.standard_normal((hkv, n_kv, d)).astype(dtype)
    v = rng.standard_normal((hkv, n_kv, d)).astype(dtype)
    pos = np.arange(n_kv - nq, n_kv, dtype=np.int32)
    return q, k, v, pos


def _visible_set(pos, n_kv, window, sinks):
    """The visible keys of a query at `pos`, enumerated as sets (reading of the
    ferrox-core windowed / sinks variants: the last `window` keys up to and
    including the query, plus the first `sinks` keys)."""
    if window <= 0:
        return set(range(pos + 1))
    return set(range(max(0, pos - window + 1), pos + 1)) | set(range(min(sinks, pos + 1)))


def _sdpa_reference(q, k, v, pos, head_map, scale, window=0, sinks=0):
    """torch fp64 scaled_dot_product_attention with an explicit boolean mask
    (no is_causal: torch's built-in causal mask is aligned top-left, while
    cache-backed queries are the suffix of the history)."""
    nq, hq, d = q.shape
    n_kv = k.shape[1]
    mask = np.zeros((nq, n_kv), bool)
    for i in range(nq):
        mask[i, sorted(_visible_set(int(pos[i]), n_kv, window, sinks))] = True
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)            # [hq][nq][d]
    kt = torch.from_numpy(k.astype(np.float64))[torch.from_numpy(head_map.astype(np.int64))]
    vt = torch.from_numpy(v.astype(np.float64))[torch.from_numpy(head_map.astype(np.int64))]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale)
    return out.permute(1, 0, 2).numpy()


# ---------------------------------------------------------- Philox / regen

@pytest.fixture(scope="session")
def rocrand_kat(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND known-answer helper")
    exe = str(tmp_path_factory.mktemp("kat") / "kat")
    subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950",
                    os.path.join(HERE, "philox_rocrand_kat.cpp"), "-o", exe], check=True,
                   capture_output=True)

    def run(rows):
        text = "\n".join(" ".join(str(int(x)) for x in r) for r in rows) + "\n"
        res = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
        return np.array([[int(t) for t in line.split()] for line in res.stdout.strip().splitlines()],
                        dtype=np.uint64).astype(np.uint32)
    return run


def test_philox_matches_rocrand(rocrand_kat):
    """Bit-exact against rocRAND's Philox4x32-10 rounds: catches a wrong
    multiplier, Weyl constant, word order or round count."""
    rng = np.random.default_rng(7)
    rows = rng.integers(0, 2**32, size=(2000, 6), dtype=np.uint64)
    rows[0] = 0
    rows[1] = 2**32 - 1
    rows[2, :4] = 0
    want = rocrand_kat(rows)
    got = np.concatenate([oracle.philox4x32_10(r[None, :4], r[4:]) for r in rows])
    np.testing.assert_array_equal(got, want)


def _uniform_from_word(x):
    return ((np.asarray(x, np.uint64) >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def test_regen_box_muller_pairing(rocrand_kat):
    """Box-Muller structure on rocRAND's words: dims 4k,4k+1 share the radius
    from word 0 and the angle from word 1; dims 4k+2,4k+3 use words 2 and 3
    (z_c^2 + z_s^2 = -2 ln u_r and atan2(z_s, z_c) = 2 pi u_a).  Catches a
    swapped sine/cosine, a wrong word pairing, or a wrong counter layout."""
    seed, layer, seq, tensor, head = 0x1234_5678_9ABC_DEF0, 3, 5, 2, 6
    for token, k4 in [(0, 0), (17, 3), (65535, 31), (123456, 7)]:
        ctr = [token, k4, head | (tensor << 30), layer | (seq << 16)]
        words = rocrand_kat([ctr + [seed & 0xFFFFFFFF, seed >> 32]])[0]
        z = [oracle.regen_value(seed, layer, seq, tensor, head, token, 4 * k4 + j) for j in range(4)]
        for pair in (0, 1):
            zc, zs = z[2 * pair], z[2 * pair + 1]
            u_r = _uniform_from_word(words[2 * pair])
            u_a = _uniform_from_word(words[2 * pair + 1])
            assert math.isclose(zc * zc + zs * zs, -2.0 * math.log(u_r), rel_tol=1e-12)
            ang = math.atan2(zs, zc) / (2 * math.pi) % 1.0
            assert math.isclose(ang, u_a, abs_tol=1e-12) or math.isclose(abs(ang - u_a), 1.0,
                                                                          abs_tol=1e-12)


def test_uniform_grid_is_exact_in_fp32():
    """Every uniform on the (x>>9 + 1/2) 2^-23 grid is an fp32 value strictly
    inside (0, 1), so an fp32 implementation sees the same u."""
    x = np.array([0, 1, 511, 512, 2**31, 2**32 - 512, 2**32 - 1], np.uint64)
    u = _uniform_from_word(x)
    assert np.all(u > 0) and np.all(u < 1)
    np.testing.assert_array_equal(u.astype(np.float32).astype(np.float64), u)


def test_regen_rounding_and_layout():
    """fp32 rows are the fp64 values rounded by numpy's RNE cast; bf16 rows are
    torch's RNE rounding of those fp32 values; rows are K[token][dim] with any
    token offset."""
    args = (42, 1, 2, 1, 3)
    f64 = oracle.regen_rows(*args, 100, 24, 128, "f64")
    f32 = oracle.regen_rows(*args, 100, 24, 128, "f32")
    b16 = oracle.regen_rows(*args, 100, 24, 128, "bf16")
    np.testing.assert_array_equal(f32, f64.astype(np.float32))
    want = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b16, want)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f32(b16),
                                  torch.from_numpy(f32).to(torch.bfloat16).float().numpy())
    sub = oracle.regen_rows(*args, 105, 3, 128, "f64")
    np.testing.assert_array_equal(sub, f64[5:8])
    assert f64[7, 77] == oracle.regen_value(*args, 107, 77)


def test_regen_streams_are_distinct():
    """Seed, layer, sequence, tensor and head each select a different stream."""
    base = (9, 0, 0, 1, 0)
    ref = oracle.regen_rows(*base, 0, 4, 64, "f64")
    for idx, alt in [(0, 10), (1, 1), (2, 1), (3, 2), (4, 1)]:
        args = list(base)
        args[idx] = alt
        other = oracle.regen_rows(*args, 0, 4, 64, "f64")
        assert not np.any(other == ref), f"argument {idx} does not change the stream"


def test_regen_is_standard_normal():
    """Moments and a Kolmogorov-Smirnov test on 2^20 values."""
    z = oracle.regen_rows(3, 0, 1, 1, 2, 0, 16384, 64, "f64").ravel()
    n = z.size
    assert abs(z.mean()) < 5.0 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5.0 * math.sqrt(2.0 / n)
    assert stats.kstest(z, "norm").pvalue > 1e-4
    zz = z.reshape(-1, 2)
    assert abs(np.corrcoef(zz[:, 0], zz[:, 1])[0, 1]) < 5.0 / math.sqrt(zz.shape[0])


# --------------------------------------------------------------- attention

@pytest.mark.parametrize("nq,n_kv,hq,hkv,d,window,sinks", [
    (1, 1, 1, 1, 64, 0, 0),
    (1, 37, 4, 4, 64, 0, 0),        # MHA
    (3, 50, 8, 1, 32, 0, 0),        # MQA
    (16, 256, 8, 2, 64, 0, 0),      # GQA, the CPUAttn parallel example's shape
    (5, 70, 6, 3, 16, 9, 0),        # window
    (5, 70, 6, 3, 16, 9, 4),        # window + sinks
    (40, 40, 2, 1, 8, 3, 2),        # full prefill, tiny window
])
def test_matches_torch_sdpa(nq, n_kv, hq, hkv, d, window, sinks):
    """fp64 agreement with torch's SDPA under an explicit mask: catches a wrong
    scale, a dropped max-subtraction error, a transposed operand or a wrong
    GQA grouping (torch's enable_gqa grouping is contiguous, h // (hq/hkv))."""
    rng = np.random.default_rng(nq * 1000 + n_kv)
    q, k, v, pos = _case(rng, nq, n_kv, hq, hkv, d)
    hm = oracle.default_head_map(hq, hkv)
    scale = 1.0 / math.sqrt(d)
    out, lse = oracle.attend(q, k, v, pos, hm, scale, window, sinks)
    np.testing.assert_allclose(out, _sdpa_reference(q, k, v, pos, hm, scale, window, sinks),
                               rtol=1e-12, atol=1e-12)
    if window == 0:
        qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)
        kt = torch.from_numpy(k.astype(np.float64))
        vt = torch.from_numpy(v.astype(np.float64))
        mask = torch.from_numpy(np.arange(n_kv)[None, :] <= pos[:, None])
        gqa = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                               scale=scale, enable_gqa=True)
        np.testing.assert_allclose(out, gqa.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    # log-sum-exp of the visible scores, via scipy
    for i in range(nq):
        vis = sorted(_visible_set(int(pos[i]), n_kv, window, sinks))
        for h in range(hq):
            s = scale * (k[hm[h], vis].astype(np.float64) @ q[i, h].astype(np.float64))
            assert math.isclose(lse[i, h], special.logsumexp(s), rel_tol=1e-12, abs_tol=1e-12)


def test_custom_head_map():
    """An arbitrary q-head -> K/V-head map: each q-head equals single-head
    attention against its own K/V head."""
    rng = np.random.default_rng(11)
    q, k, v, pos = _case(rng, 4, 30, 6, 3, 16)
    hm = np.array([2, 0, 1, 1, 0, 2], np.int32)
    out, _ = oracle.attend(q, k, v, pos, hm, 0.3)
    for h in range(6):
        single, _ = oracle.attend(q[:, h:h + 1], k[hm[h]:hm[h] + 1], v[hm[h]:hm[h] + 1], pos,
                                  np.zeros(1, np.int32), 0.3)
        np.testing.assert_array_equal(out[:, h], single[:, 0])
        ref = _sdpa_reference(q[:, h:h + 1], k[hm[h]:hm[h] + 1], v[hm[h]:hm[h] + 1], pos,
                              np.zeros(1, np.int32), 0.3)
        np.testing.assert_allclose(out[:, h:h + 1], ref, rtol=1e-12, atol=1e-12)


def test_single_visible_key_returns_that_row():
    """One visible key: the output is that V row exactly (the history of one
    token, and a window of one without sinks at any position)."""
    rng = np.random.default_rng(1)
    q, k, v, pos = _case(rng, 1, 1, 2, 1, 64)
    out, lse = oracle.attend(q, k, v, pos, np.zeros(2, np.int32), 0.125)
    np.testing.assert_array_equal(out[0, 0], v[0, 0].astype(np.float64))
    np.testing.assert_array_equal(out[0, 1], v[0, 0].astype(np.float64))
    assert math.isclose(lse[0, 0], 0.125 * float(q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64)),
                        rel_tol=1e-13)
    q, k, v, pos = _case(rng, 12, 12, 1, 1, 8)
    out, _ = oracle.attend(q, k, v, pos, np.zeros(1, np.int32), 1.0, window=1)
    np.testing.assert_array_equal(out[:, 0], v[0].astype(np.float64))


@pytest.mark.parametrize("window,sinks", [(0, 0), (1, 0), (1, 3), (4, 2), (7, 0), (100, 5), (3, 50)])
def test_identical_keys_average_exactly_the_visible_values(window, sinks):
    """With every key equal, the weights are uniform, so each output row is the
    mean of V over the visible set and lse = s + ln |visible|.  This pins the
    window and sink semantics (off-by-one in the window, sinks counted twice,
    sinks beyond the query) independently of the softmax arithmetic."""
    rng = np.random.default_rng(window * 10 + sinks)
    n_kv, d = 23, 8
    q = rng.standard_normal((n_kv, 1, d)).astype(np.float32)
    krow = rng.standard_normal(d).astype(np.float32)
    k = np.broadcast_to(krow, (1, n_kv, d)).copy()
    v = rng.standard_normal((1, n_kv, d)).astype(np.float32)
    pos = np.arange(n_kv, dtype=np.int32)
    out, lse = oracle.attend(q, k, v, pos, np.zeros(1, np.int32), 0.5, window, sinks)
    for i in range(n_kv):
        vis = sorted(_visible_set(i, n_kv, window, sinks))
        np.testing.assert_allclose(out[i, 0], v[0, vis].astype(np.float64).mean(axis=0),
                                   rtol=1e-13, atol=1e-14)
        s = 0.5 * float(q[i, 0].astype(np.float64) @ krow.astype(np.float64))
        assert math.isclose(lse[i, 0], s + math.log(len(vis)), rel_tol=1e-13, abs_tol=1e-13)


def test_two_keys_closed_form():
    """Two visible keys: o = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1."""
    rng = np.random.default_rng(5)
    q, k, v, pos = _case(rng, 1, 2, 1, 1, 16)
    out, _ = oracle.attend(q, k, v, pos, np.zeros(1, np.int32), 0.7)
    s = 0.7 * (k[0].astype(np.float64) @ q[0, 0].astype(np.float64))
    want = special.expit(s[0] - s[1]) * v[0, 0] + special.expit(s[1] - s[0]) * v[0, 1]
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-13, atol=1e-14)


def test_softcap_closed_form():
    """Softcap c on two keys whose scaled scores are c*atanh(t0), c*atanh(t1):
    the capped scores are exactly c*t0 and c*t1.  Catches capping before the
    scale, a missing outer factor c, or capping after the softmax."""
    cap, scale = 2.0, 0.25
    t = np.array([0.5, -0.25])
    raw = cap * np.arctanh(t)                    # wanted scaled scores
    q = np.zeros((1, 1, 2), np.float32)
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 2, 2), np.float32)
    k[0, :, 0] = (raw / scale).astype(np.float32)
    v = np.array([[[1.0, 3.0], [-2.0, 0.5]]], np.float32)
    out, lse = oracle.attend(q, k, v, np.array([1], np.int32), np.zeros(1, np.int32), scale,
                             softcap=cap)
    capped = cap * np.tanh(scale * k[0, :, 0].astype(np.float64) / cap)
    assert np.allclose(capped, cap * t, atol=1e-7)   # float32 storage of the designed scores
    want = special.expit(capped[0] - capped[1]) * v[0, 0] + special.expit(capped[1] - capped[0]) * v[0, 1]
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-12, atol=1e-13)
    assert math.isclose(lse[0, 0], special.logsumexp(capped), rel_tol=1e-13)
    # without the cap the same inputs give a different answer
    plain, _ = oracle.attend(q, k, v, np.array([1], np.int32), np.zeros(1, np.int32), scale)
    assert np.max(np.abs(plain - out)) > 1e-2


def test_limits_reduce_to_plain_causal():
    """softcap -> infinity and window >= history both reduce to plain causal."""
    rng = np.random.default_rng(8)
    q, k, v, pos = _case(rng, 6, 40, 4, 2, 32)
    hm = oracle.default_head_map(4, 2)
    plain, plse = oracle.attend(q, k, v, pos, hm, 0.2)
    capped, clse = oracle.attend(q, k, v, pos, hm, 0.2, softcap=1e30)
    np.testing.assert_allclose(capped, plain, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(clse, plse, rtol=1e-12, atol=1e-12)
    wide, _ = oracle.attend(q, k, v, pos, hm, 0.2, window=40, n_sinks=3)
    np.testing.assert_array_equal(wide, plain)


def test_scale_invariance_and_convex_hull():
    """q*c with scale/c gives the same output, and every output lies inside the
    per-dimension range of the visible V rows."""
    rng = np.random.default_rng(9)
    q, k, v, pos = _case(rng, 8, 33, 4, 4, 16)
    hm = oracle.default_head_map(4, 4)
    a, _ = oracle.attend(q, k, v, pos, hm, 0.5)
    b, _ = oracle.attend(q * np.float32(4.0), k, v, pos, hm, 0.125)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    for i in range(8):
        vis = v[:, : pos[i] + 1].astype(np.float64)
        lo, hi = vis.min(axis=1), vis.max(axis=1)
        assert np.all(a[i] >= lo - 1e-12) and np.all(a[i] <= hi + 1e-12)


def test_permutation_invariance_of_the_full_history():
    """The last query sees every key: permuting the K/V rows jointly leaves its
    output unchanged (the history is a set, not a sequence, to softmax)."""
    rng = np.random.default_rng(10)
    q, k, v, pos = _case(rng, 1, 64, 2, 1, 16)
    perm = rng.permutation(64)
    a, la = oracle.attend(q, k, v, pos, np.zeros(2, np.int32), 0.3)
    b, lb = oracle.attend(q, k[:, perm], v[:, perm], pos, np.zeros(2, np.int32), 0.3)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=1e-13)


def test_folded_pages_equal_full_kv():
    """CFR-Atlas "Core contract": folding the history page by page into a
    running (max, sum, acc) state and merging gives full-KV attention.  The
    fold here is test-only fp64 numpy (not the oracle), over random page
    partitions and merge orders."""
    rng = np.random.default_rng(12)
    q, k, v, pos = _case(rng, 1, 300, 1, 1, 32)
    want, wlse = oracle.attend(q, k, v, pos, np.zeros(1, np.int32), 0.2)
    qd = q[0, 0].astype(np.float64)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, 300), size=rng.integers(1, 20), replace=False))
        bounds = [0, *cuts.tolist(), 300]
        parts = []
        for a, b in zip(bounds[:-1], bounds[1:]):
            s = 0.2 * (k[0, a:b].astype(np.float64) @ qd)
            m = s.max()
            p = np.exp(s - m)
            parts.append((m, p.sum(), p @ v[0, a:b].astype(np.float64)))
        order = rng.permutation(len(parts))
        m, l, acc = -np.inf, 0.0, np.zeros(32)
        for idx in order:
            pm, pl, pacc = parts[idx]
            nm = max(m, pm)
            l = l * math.exp(m - nm) + pl * math.exp(pm - nm)
            acc = acc * math.exp(m - nm) + pacc * math.exp(pm - nm)
            m = nm
        np.testing.assert_allclose(acc / l, want[0, 0], rtol=1e-12, atol=1e-13)
        assert math.isclose(m + math.log(l), wlse[0, 0], rel_tol=1e-13)


def test_gather_pages_unpages_a_shuffled_arena():
    """The paged->unpaged gather used by the tests returns rows in logical
    order whatever the physical placement."""
    rng = np.random.default_rng(13)
    P, H, D, n = 4, 2, 3, 13
    rows = rng.standard_normal((H, 16, D))
    perm = rng.permutation(6)
    arena = np.full((6, H, P, D), np.nan)
    for lp in range(4):
        arena[perm[lp]] = rows[:, lp * P:(lp + 1) * P].reshape(H, P, D)
    got = oracle.gather_pages(arena, perm, n, P)
    np.testing.assert_array_equal(got, rows[:, :n])


def test_rejects_empty_or_out_of_range():
    rng = np.random.default_rng(14)
    q, k, v, pos = _case(rng, 1, 4, 1, 1, 4)
    with pytest.raises(ValueError):
        oracle.attend(q, k, v, np.array([4], np.int32), np.zeros(1, np.int32), 1.0)
    with pytest.raises(ValueError):
        oracle.attend(q, k, v, pos, np.array([1], np.int32), 1.0)
