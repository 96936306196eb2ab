"""Pins for the oracle's attention over several new tokens per sequence
(``oracle.multi_token``): torch's own attention with an explicit causal mask on the
logical K/V (never through a table), the one-token case against the decode oracle,
causality (a token's output ignores every later position), and the closed form of
equal keys (the mean of the visible values).  CPU only.

Pages: [ASP] "PagedAttention" (awesome-system-papers), 实现要点 (continuous
batching) and 已知局限 (speculative decoding), 引用本概念的论文 (the scaled dot-product
attention the cache serves)."""
import numpy as np
import pytest
import torch

from tests.helpers import place, table_array
from tests.test_oracle_pins import _rand


def _case(rng, lens, new, Hq, Hkv, D, bs, dtype, gain=1.0, extra_blocks=3):
    """Logical K/V per sequence in a shuffled pool; queries for the last new[s] tokens."""
    nb = [(L + bs - 1) // bs for L in lens]
    N = sum(nb) + extra_blocks
    perm = rng.permutation(N)
    rows, at = [], 0
    for n in nb:
        rows.append(perm[at:at + n].tolist())
        at += n
    ks = [_rand(rng, (L, Hkv, D), dtype) for L in lens]
    vs = [_rand(rng, (L, Hkv, D), dtype) for L in lens]
    kc, vc = place(ks, vs, rows, N, bs, dtype)
    qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    q = _rand(rng, (int(qs[-1]), Hq, D), dtype, gain)
    bt = table_array(rows, max(max(nb), 1) + 2)
    return q, ks, vs, kc, vc, bt, np.asarray(lens, np.int32), qs


def _torch_causal(q64, K64, V64, ctx, scale):
    """torch SDPA in fp64: q [n, Hq, D] at positions ctx .. ctx+n-1 over K/V [L, Hkv, D]."""
    n, Hq, _ = q64.shape
    L, Hkv, _ = K64.shape
    G = Hq // Hkv
    qt = torch.from_numpy(np.ascontiguousarray(q64.transpose(1, 0, 2)))[None]      # [1, Hq, n, D]
    kt = torch.from_numpy(np.ascontiguousarray(K64.transpose(1, 0, 2)))[None].repeat_interleave(G, 1)
    vt = torch.from_numpy(np.ascontiguousarray(V64.transpose(1, 0, 2)))[None].repeat_interleave(G, 1)
    mask = torch.arange(L)[None, :] <= (ctx + torch.arange(n))[:, None]            # [n, L]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("Hq,Hkv,bs", [(4, 4, 4), (8, 2, 16), (6, 1, 8)])
def test_multi_token_equals_torch_causal_sdpa(oracle_mod, dtype, Hq, Hkv, bs):
    rng = np.random.default_rng(Hq * 100 + bs)
    lens, new = [9, 40, 33, 17], [9, 5, 1, 16]     # a whole prompt, chunks, one token
    D = 16
    q, ks, vs, kc, vc, bt, sl, qs = _case(rng, lens, new, Hq, Hkv, D, bs, dtype)
    got = oracle_mod.multi_token(q, kc, vc, bt, sl, qs, bs, Hkv, 0.3, dtype)
    dec = lambda a: oracle_mod.decode_elements(a, dtype)  # noqa: E731
    for s, (L, n) in enumerate(zip(lens, new)):
        want = _torch_causal(dec(q[qs[s]:qs[s + 1]]), dec(ks[s]), dec(vs[s]), L - n, 0.3)
        np.testing.assert_allclose(got[qs[s]:qs[s + 1]], want, rtol=1e-12, atol=1e-13)


def test_one_new_token_is_decode(oracle_mod):
    rng = np.random.default_rng(7)
    lens = [1, 5, 16, 17, 100]
    q, ks, vs, kc, vc, bt, sl, qs = _case(rng, lens, [1] * 5, 8, 2, 32, 4, "bf16")
    got = oracle_mod.multi_token(q, kc, vc, bt, sl, qs, 4, 2, 0.2, "bf16")
    want = oracle_mod.decode(q, kc, vc, bt, sl, 4, 2, 0.2, "bf16")
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)


def test_later_positions_are_never_seen(oracle_mod):
    """Overwrite the last cached token with huge values: every earlier new token's
    output stays bit-identical, the last one's changes."""
    rng = np.random.default_rng(8)
    lens, new = [30, 12], [6, 12]
    q, ks, vs, kc, vc, bt, sl, qs = _case(rng, lens, new, 4, 2, 16, 4, "f32")
    before = oracle_mod.multi_token(q, kc, vc, bt, sl, qs, 4, 2, 0.25, "f32")
    for s, L in enumerate(lens):
        ks[s][L - 1] = 1e4
        vs[s][L - 1] = -1e4
    kc2, vc2 = place(ks, vs, [[b for b in r if b >= 0] for r in bt.tolist()], kc.shape[0], 4, "f32")
    after = oracle_mod.multi_token(q, kc2, vc2, bt, sl, qs, 4, 2, 0.25, "f32")
    for s in range(2):
        last = qs[s + 1] - 1
        np.testing.assert_array_equal(after[qs[s]:last], before[qs[s]:last])
        assert np.abs(after[last] - before[last]).max() > 1.0


def test_equal_keys_give_the_running_mean(oracle_mod):
    """A whole prompt (no context) with every key equal: token j's output is the
    mean of V[0 .. j] -- off by one position either way fails."""
    rng = np.random.default_rng(9)
    L, Hkv, D, bs = 13, 1, 8, 4
    k = np.repeat(_rand(rng, (1, Hkv, D), "f32"), L, axis=0)
    v = _rand(rng, (L, Hkv, D), "f32")
    rows = [list(rng.permutation(6)[:4])]
    kc, vc = place([k], [v], rows, 6, bs, "f32")
    q = _rand(rng, (L, 2, D), "f32")
    got = oracle_mod.multi_token(q, kc, vc, table_array(rows, 4), np.array([L], np.int32),
                                 np.array([0, L], np.int32), bs, Hkv, 1.0, "f32")
    v64 = v.astype(np.float64)[:, 0, :]
    for j in range(L):
        want = v64[:j + 1].mean(axis=0)
        for h in range(2):
            np.testing.assert_allclose(got[j, h], want, rtol=1e-12, atol=1e-14)


def test_empty_chunks_and_errors(oracle_mod):
    rng = np.random.default_rng(10)
    q, ks, vs, kc, vc, bt, sl, qs = _case(rng, [5, 7], [0, 3], 2, 2, 8, 4, "f32")
    out = oracle_mod.multi_token(q, kc, vc, bt, sl, qs, 4, 2, 0.5, "f32")
    assert out.shape == (3, 2, 8) and np.isfinite(out).all()
    with pytest.raises(oracle_mod.OracleError) as e:       # more new tokens than cached
        oracle_mod.multi_token(q, kc, vc, bt, np.array([5, 2], np.int32), qs, 4, 2, 0.5, "f32")
    assert e.value.code == oracle_mod.BAD_LEN
    with pytest.raises(oracle_mod.OracleError) as e:       # query_start not ending at T
        oracle_mod.multi_token(q, kc, vc, bt, sl, np.array([0, 0, 2], np.int32), 4, 2, 0.5, "f32")
    assert e.value.code == oracle_mod.BAD_ARG
    bad = bt.copy()
    bad[1, 0] = kc.shape[0]
    with pytest.raises(oracle_mod.OracleError) as e:
        oracle_mod.multi_token(q, kc, vc, bad, sl, qs, 4, 2, 0.5, "f32")
    assert e.value.code == oracle_mod.BAD_BLOCK
