"""Pins of the prefill oracle (oracle.prefill) against facts that do not come from it:
torch's scaled_dot_product_attention with an explicit causal mask, the scalar-loop
decode reference (a prefill token at position p is a decode over positions 0..p),
causality, and the first-token closed form; plus planted mistakes that the pins
must catch."""
import numpy as np
import pytest

import oracle
import oracle.prefill as opf
import workloads
from oracle.numerics import bits_to_f64
from oracle_pins import make_case


def _case(Hq, Hkv, D, bs, lens, new, dtype="bf16", seed=0):
    """Pools holding known contexts (make_case) and new-token queries: the last new[i]
    positions of sequence i."""
    case = make_case(Hq, Hkv, D, bs, lens, dtype=dtype, seed=seed)
    rng = np.random.default_rng(seed + 31)
    qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int64)
    q = workloads.random_bits(rng, (int(qs[-1]), Hq, D), dtype)
    return case, q, qs


def _run(fn, case, q, qs, **kw):
    c = case.cfg
    args = dict(k_cache=case.k_cache, v_cache=case.v_cache, block_tables=case.wl.block_tables,
                context_lens=case.wl.context_lens)
    args.update(kw)
    return fn(q, args["k_cache"], args["v_cache"], args["block_tables"], args["context_lens"], qs, c.scale,
              dtype=c.dtype, num_blocks=case.wl.num_blocks, num_kv_heads=c.num_kv_heads, block_size=c.block_size)


SHAPES = [("bf16", 8, 2, 64, 16, [37, 64, 100, 5], [37, 20, 1, 5]),
          ("fp16", 4, 4, 128, 16, [33, 16], [10, 16]),
          ("bf16", 16, 1, 64, 256, [300, 257], [300, 3])]


def pin_library_sdpa(fn):
    """torch's scaled_dot_product_attention in float64 with an explicit boolean mask
    (query j sees keys 0 .. L - n + j) and its own GQA convention."""
    import torch
    import torch.nn.functional as F
    for k, (dtype, Hq, Hkv, D, bs, lens, new) in enumerate(SHAPES):
        case, q, qs = _case(Hq, Hkv, D, bs, lens, new, dtype, seed=40 + k)
        out = _run(fn, case, q, qs)
        qf = bits_to_f64(q, dtype)
        for i, (L, n) in enumerate(zip(lens, new)):
            kk = torch.from_numpy(bits_to_f64(case.ctx_k[i], dtype)).permute(1, 0, 2)[None]   # [1,Hkv,L,D]
            vv = torch.from_numpy(bits_to_f64(case.ctx_v[i], dtype)).permute(1, 0, 2)[None]
            qq = torch.from_numpy(qf[qs[i]:qs[i + 1]]).permute(1, 0, 2)[None]                 # [1,Hq,n,D]
            mask = torch.from_numpy(np.arange(L)[None, :] <= (L - n + np.arange(n))[:, None])
            ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=case.cfg.scale, enable_gqa=True)
            np.testing.assert_allclose(out[qs[i]:qs[i + 1]], ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def pin_scalar_decode_per_position(fn):
    """New token j of sequence i equals the scalar-loop decode of that one query over a
    context of L - n + j + 1 positions (same pool, same table)."""
    case, q, qs = _case(4, 2, 16, 16, [21, 40], [21, 6], "bf16", seed=7)
    out = _run(fn, case, q, qs)
    c = case.cfg
    for i, (L, n) in enumerate(zip([21, 40], [21, 6])):
        for j in range(n):
            ref = oracle.brute.decode(q[qs[i] + j][None], case.k_cache, case.v_cache, case.wl.block_tables[i:i + 1],
                                      np.array([L - n + j + 1]), c.scale, dtype=c.dtype,
                                      num_kv_heads=c.num_kv_heads, block_size=c.block_size)
            np.testing.assert_allclose(out[qs[i] + j], ref[0], rtol=1e-12, atol=1e-12)


def pin_last_token_is_decode(fn):
    """The last new token of each sequence sees the whole context: the decode oracle."""
    dtype, Hq, Hkv, D, bs, lens, new = SHAPES[0]
    case, q, qs = _case(Hq, Hkv, D, bs, lens, new, dtype, seed=9)
    out = _run(fn, case, q, qs)
    last = q[qs[1:] - 1]
    c = case.cfg
    ref = oracle.decode(last, case.k_cache, case.v_cache, case.wl.block_tables, case.wl.context_lens, c.scale,
                        dtype=c.dtype, num_blocks=case.wl.num_blocks, num_kv_heads=Hkv, block_size=bs)
    np.testing.assert_allclose(out[qs[1:] - 1], ref, rtol=1e-12, atol=1e-12)


def pin_causality(fn):
    """Changing the K/V of later positions leaves every earlier token's output bit-identical,
    and changes the token that sees them."""
    Hq, Hkv, D, bs, L = 4, 2, 16, 16, 30
    case, q, qs = _case(Hq, Hkv, D, bs, [L], [L], "bf16", seed=11)
    base = _run(fn, case, q, qs)
    p = 17
    k2 = [c.copy() for c in case.ctx_k]
    v2 = [c.copy() for c in case.ctx_v]
    rng = np.random.default_rng(3)
    k2[0][p + 1:] = workloads.random_bits(rng, k2[0][p + 1:].shape, "bf16")
    v2[0][p + 1:] = workloads.random_bits(rng, v2[0][p + 1:].shape, "bf16")
    case2 = make_case(Hq, Hkv, D, bs, [L], dtype="bf16", seed=11, ctx_k=k2, ctx_v=v2)
    out2 = _run(fn, case2, q, qs)
    assert np.array_equal(base[:p + 1], out2[:p + 1])
    assert not np.allclose(base[p + 1], out2[p + 1])


def pin_first_token_is_v0(fn):
    """With no prefix, the first new token sees only position 0: its output is V_0 exactly."""
    Hq, Hkv, D = 8, 2, 64
    case, q, qs = _case(Hq, Hkv, D, 16, [12, 50], [12, 50], "fp16", seed=13)
    out = _run(fn, case, q, qs)
    for i in range(2):
        v0 = bits_to_f64(case.ctx_v[i][0], "fp16")
        for h in range(Hq):
            assert np.array_equal(out[qs[i], h], v0[h // (Hq // Hkv)])


def pin_empty_sequences(fn):
    """A sequence with no new tokens contributes no rows and leaves the others unchanged."""
    case, q, qs = _case(4, 2, 16, 16, [10, 20, 15], [4, 0, 15], "bf16", seed=17)
    out = _run(fn, case, q, qs)
    assert out.shape[0] == 19
    one = make_case(4, 2, 16, 16, [10], dtype="bf16", seed=17)
    alone = _run(fn, one, q[:4], np.array([0, 4]))
    assert np.array_equal(alone, out[:4])


ALL_PINS = [pin_library_sdpa, pin_scalar_decode_per_position, pin_last_token_is_decode, pin_causality,
            pin_first_token_is_v0, pin_empty_sequences]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_prefill_oracle_pin(pin):
    pin(opf.prefill)


MUTANTS = {
    "sees-one-more": lambda mp: mp.setattr(opf, "visible_keys", lambda p: p + 2),
    "sees-one-less": lambda mp: mp.setattr(opf, "visible_keys", lambda p: max(p, 1)),
    "ignores-prefix": lambda mp: mp.setattr(opf, "position_of", lambda L, n, j: j),
    "sees-everything": lambda mp: mp.setattr(opf, "position_of", lambda L, n, j: L - 1),
    "gqa-modulo": lambda mp: mp.setattr(opf, "kv_head_of", lambda h, g: h % 2),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(opf.prefill)
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
