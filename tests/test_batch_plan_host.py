"""Batch-size dispatch planner (pi_batch_plan), host only.

The expected per-token count n and union U of B independent tokens are pinned against an
exhaustive enumeration of every outcome on a tiny layer and against a Monte-Carlo draw of
token masks; the choice against the cases the model fixes (one token, int4 weights, a
heavy overlap of the tokens' lists)."""
import itertools
import math

import numpy as np
import pytest

from activation_sparse_pi_amd import _lib as L

A = 0x7F0000000000


def ffn(d=8192, F=64, act=L.PI_ACT_RELU, wfmt=L.PI_W_F16):
    s = A + 0x2000000 if wfmt == L.PI_W_I4G128 else None
    g = A + 0x3000000 if act == L.PI_ACT_REGLU else None
    return L.FfnDesc(g, A, A + 0x1000000, s if g else None, s, s, d, F, act, wfmt)


def plan(rate, B, desc=None, hbm=8000.0):
    rate = np.ascontiguousarray(rate, dtype=np.float32)
    desc = desc or ffn(F=rate.size)
    p = L.BatchPlan()
    st = L.pi_batch_plan(desc, B, rate.ctypes.data, hbm, p)
    assert st == L.PI_OK, L.pi_last_error()
    return p


def test_expected_union_by_enumeration():
    """Tiny layer: E[union] and E[n] by summing over every joint outcome of B tokens."""
    rate = np.array([0.5, 0.25, 0.75, 0.0, 1.0, 0.125, 0.5, 0.625], np.float32)
    F, B = rate.size, 2
    eu = en = 0.0
    for bits in itertools.product((0, 1), repeat=F * B):
        m = np.array(bits).reshape(B, F)
        pr = np.prod(np.where(m == 1, rate[None, :], 1.0 - rate[None, :]))
        eu += pr * m.any(axis=0).sum()
        en += pr * m[0].sum()
    p = plan(rate, B)
    assert p.u_mean == pytest.approx(eu, rel=1e-12, abs=1e-12)
    assert p.n_mean == pytest.approx(en, rel=1e-12, abs=1e-12)


def test_expected_union_by_sampling():
    rng = np.random.default_rng(7)
    F, B, T = 512, 12, 4000
    rate = np.clip(rng.gamma(0.6, 0.12, F), 0.0, 1.0).astype(np.float32)
    masks = rng.random((T, B, F)) < rate[None, None, :]
    u = masks.any(axis=1).sum(axis=1)
    p = plan(rate, B)
    sem = u.std() / math.sqrt(T)
    assert abs(u.mean() - p.u_mean) < 5 * sem
    assert abs(masks[:, 0].sum(axis=1).mean() - p.n_mean) < 5 * masks[:, 0].sum(axis=1).std() / math.sqrt(T)


def test_one_token_and_int4_take_the_token_path():
    rate = np.full(256, 0.1, np.float32)
    p1 = plan(rate, 1)
    assert p1.choice == L.PI_BATCH_TOKENS and math.isinf(p1.t_union_us)
    assert p1.u_mean == pytest.approx(p1.n_mean, rel=1e-12)
    p4 = plan(rate, 8, ffn(F=256, wfmt=L.PI_W_I4G128))
    assert p4.choice == L.PI_BATCH_TOKENS and math.isinf(p4.t_union_us)


def test_overlap_decides():
    """Identical lists (rates 0 or 1): the union pass reads one token's rows for all B tokens,
    so once B tokens' rows outweigh the union pass's larger fixed cost it wins, and it keeps
    winning as B grows; sparse, barely overlapping lists stay on the token path."""
    F = 32768
    rate = np.zeros(F, np.float32)
    rate[:2600] = 1.0
    picks = []
    for B in (2, 4, 8, 16, 32):
        p = plan(rate, B, ffn(F=F))
        assert p.u_mean == pytest.approx(2600)
        # the union's estimate does not grow with B (one pass), the tokens' grows linearly
        picks.append(p.choice)
    assert picks[-1] == L.PI_BATCH_UNION
    first = picks.index(L.PI_BATCH_UNION)
    assert all(c == L.PI_BATCH_UNION for c in picks[first:]), picks
    sparse = np.full(F, 4.0 / F, np.float32)            # ~4 neurons per token
    q = plan(sparse, 2, ffn(F=F))
    assert q.choice == L.PI_BATCH_TOKENS


def test_token_time_is_linear_in_batch():
    rate = np.full(1024, 0.05, np.float32)
    t = [plan(rate, B).t_tokens_us for B in (1, 2, 4, 8)]
    assert t[1] == pytest.approx(2 * t[0]) and t[3] == pytest.approx(8 * t[0])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), L.PI_ERR_SHAPE),
    (dict(B=65), L.PI_ERR_SHAPE),
    (dict(hbm=0.0), L.PI_ERR_SHAPE),
    (dict(bad=1.5), L.PI_ERR_SHAPE),
    (dict(bad=float("nan")), L.PI_ERR_SHAPE),
    (dict(bad=-0.1), L.PI_ERR_SHAPE),
    (dict(null_rate=True), L.PI_ERR_NULL),
    (dict(null_plan=True), L.PI_ERR_NULL),
    (dict(null_desc=True), L.PI_ERR_NULL),
])
def test_validation(kw, code):
    rate = np.full(64, 0.1, np.float32)
    if "bad" in kw:
        rate[5] = kw["bad"]
    p = L.BatchPlan()
    p.choice = 77
    st = L.pi_batch_plan(None if kw.get("null_desc") else ffn(F=64), kw.get("B", 4),
                         None if kw.get("null_rate") else rate.ctypes.data, kw.get("hbm", 8000.0),
                         None if kw.get("null_plan") else p)
    assert st == code, L.pi_last_error()
    assert p.choice == 77                                  # untouched on error


def test_bytes_per_row_follow_matrices_and_format():
    """The variable part of each estimate scales with the bytes of one listed neuron:
    m d w, with m = 2 (ReLU) or 3 (ReGLU) and w = 2 (fp16) or 0.5 + 2/128 (int4 g128)."""
    F, d, B = 4096, 4096, 4
    rate = np.full(F, 0.1, np.float32)
    base = plan(rate, B, ffn(d=d, F=F))
    glu = plan(rate, B, ffn(d=d, F=F, act=L.PI_ACT_REGLU))
    i4 = plan(rate, B, ffn(d=d, F=F, wfmt=L.PI_W_I4G128))
    tiny = plan(np.full(F, 1e-9, np.float32), B, ffn(d=d, F=F))    # ~ the fixed costs alone
    tok = lambda p: p.t_tokens_us - tiny.t_tokens_us                  # noqa: E731
    uni = lambda p: p.t_union_us - tiny.t_union_us                    # noqa: E731
    assert tok(glu) / tok(base) == pytest.approx(1.5, rel=1e-6)
    assert uni(glu) / uni(base) == pytest.approx(1.5, rel=1e-6)
    assert tok(i4) / tok(base) == pytest.approx((0.5 + 2 / 128) / 2, rel=1e-6)


def test_more_than_32_tokens_run_as_union_passes():
    """B > 32 is priced as ceil(B / 32) union passes of near-equal groups: 64 tokens as two
    passes of 32 (twice the 32-token union estimate), 33 as 17 + 16 (u_mean the mean of the two
    groups' expected unions); the token path stays linear in B."""
    F = 4096
    rate = np.clip(np.random.default_rng(5).gamma(0.5, 0.1, F), 0, 1).astype(np.float32)
    r64 = rate.astype(np.float64)
    eu = lambda b: float(np.sum(1.0 - (1.0 - r64) ** b))          # noqa: E731
    p32, p64 = plan(rate, 32), plan(rate, 64)
    assert p64.u_mean == pytest.approx(eu(32), rel=1e-9)
    assert p64.t_union_us == pytest.approx(2 * p32.t_union_us, rel=1e-9)
    assert p64.t_tokens_us == pytest.approx(2 * p32.t_tokens_us, rel=1e-9)
    p33, p17, p16 = plan(rate, 33), plan(rate, 17), plan(rate, 16)
    assert p33.u_mean == pytest.approx(0.5 * (eu(17) + eu(16)), rel=1e-9)
    assert p33.t_union_us == pytest.approx(p17.t_union_us + p16.t_union_us, rel=1e-9)
