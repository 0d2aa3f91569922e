"""Pins for two oracle helpers every other check leans on: the block-table
validity checker (oracle.alloc_check) and the exact 16-bit -> float64
conversion (oracle.numerics.bits_to_f64).

check_tables is pinned by hand-made tables whose validity is decided here case
by case from the paging rules ("vLLM — PagedAttention으로 ...", section
"PagedAttention — OS 가상 메모리에서 영감": a sequence holds ceil(L / bs) blocks
anywhere in the pool, no block serves two places; "Nano-vLLM로 배우는 ...",
section "KV 캐시와 Block Manager": shared prompt-prefix blocks): one valid table
and one invalid table per rule, each of which must raise.  Planted mistakes in
the checker (each rule dropped or loosened) must each let one invalid table
through.

bits_to_f64 is pinned by closed-form values of chosen bit patterns (IEEE
binary16 and bfloat16: 1, -2, the smallest subnormal, the smallest normal, the
largest finite value, infinities, signed zero) and by an exhaustive comparison
over all 65,536 patterns with a decoder written here from the bit fields
(sign, exponent, mantissa) with math.ldexp.  Planted mistakes (fp16 converted
by value instead of reinterpreted, bf16 shifted by the wrong amount, the sign
dropped) must each fail a pin.
"""
import math

import numpy as np
import pytest

from oracle import alloc_check
from oracle import numerics

BS = 4
N = 10
PAD = -1


def _valid_case():
    # seq 0: 9 tokens -> 3 blocks; seq 1: 6 tokens -> 2 blocks; seq 2: empty.
    tables = np.array([[3, 7, 0, PAD], [5, 2, PAD, PAD], [PAD, PAD, PAD, PAD]], dtype=np.int32)
    return tables, np.array([9, 6, 0], dtype=np.int32)


def _shared_case():
    # seqs 0 and 1 share block 3 as their logical block 0 (full, before every write)
    tables = np.array([[3, 7, PAD], [3, 5, 2]], dtype=np.int32)
    return tables, np.array([6, 12], dtype=np.int32)


def test_valid_tables_pass_and_count_blocks():
    t, L = _valid_case()
    assert alloc_check.check_tables(t, L, num_blocks=N, block_size=BS, pad_value=PAD) == 5
    t, L = _shared_case()
    assert alloc_check.check_tables(t, L, num_blocks=N, block_size=BS, pad_value=PAD, shared=[3]) == 4
    assert alloc_check.check_tables(t, L, num_blocks=N, block_size=BS, pad_value=PAD, shared=[3],
                                    appended=False) == 4


def _invalid_cases():
    """(name, kwargs for check_tables): every one breaks exactly one paging rule."""
    cases = []
    t, L = _valid_case()
    dup = t.copy()
    dup[1, 1] = 7                      # block 7 also seq 0's logical block 1
    cases.append(("held-twice", dict(tables=dup, lens=L)))
    dup_same_idx = t.copy()
    dup_same_idx[1, 0] = 3             # same logical index as seq 0, but not declared shared
    cases.append(("held-twice-same-index", dict(tables=dup_same_idx, lens=L)))
    hi = t.copy()
    hi[0, 2] = N                       # one past the pool
    cases.append(("id-past-pool", dict(tables=hi, lens=L)))
    neg = t.copy()
    neg[1, 0] = -2
    cases.append(("id-negative", dict(tables=neg, lens=L)))
    pad = t.copy()
    pad[1, 3] = 4                      # an entry past ceil(6/4) = 2 that is not padding
    cases.append(("padding-wrong", dict(tables=pad, lens=L)))
    cases.append(("table-too-short", dict(tables=t[:, :2], lens=L)))

    st, SL = _shared_case()
    moved = st.copy()
    moved[1] = [5, 3, 2]               # shared block 3 at logical index 1 of seq 1
    cases.append(("shared-other-index", dict(tables=moved, lens=SL, shared=[3])))
    # appended=True: position L-1 was just written, so a shared block must end at or before L-1.
    # Seq 0 with L = 4 holds block 3 as its only block, which contains position 3 = L-1.
    cases.append(("shared-holds-appended-token", dict(tables=np.array([[3, PAD, PAD], [3, 5, 2]], np.int32),
                                                      lens=np.array([4, 12], np.int32), shared=[3])))
    # appended=False: the next write is position L.  With L = 3, block 3 (positions 0..3)
    # is not full, so position 3 would be written into the shared block.
    cases.append(("shared-not-full-before-next-write",
                  dict(tables=np.array([[3, PAD, PAD], [3, 5, 2]], np.int32),
                       lens=np.array([3, 12], np.int32), shared=[3], appended=False)))
    # Same tables, appended=True: L = 3 means position 2 was written into block 3.
    cases.append(("shared-appended-into",
                  dict(tables=np.array([[3, PAD, PAD], [3, 5, 2]], np.int32),
                       lens=np.array([3, 12], np.int32), shared=[3])))
    return cases


def _run(check, kw):
    kw = dict(kw)
    return check(kw.pop("tables"), kw.pop("lens"), num_blocks=N, block_size=BS, pad_value=PAD, **kw)


@pytest.mark.parametrize("name,kw", _invalid_cases(), ids=[c[0] for c in _invalid_cases()])
def test_invalid_table_is_rejected(name, kw):
    with pytest.raises(AssertionError):
        _run(alloc_check.check_tables, kw)


def test_boundary_full_shared_block_is_accepted():
    # appended=False with L = 4: block 3 (positions 0..3) is full and the next write is 4
    t = np.array([[3, PAD, PAD], [3, 5, 2]], np.int32)
    alloc_check.check_tables(t, np.array([4, 12], np.int32), num_blocks=N, block_size=BS,
                             pad_value=PAD, shared=[3], appended=False)
    # appended=True with L = 5: position 4 (block 1) was written, block 3 ends before it
    t = np.array([[3, 6, PAD], [3, 5, 2]], np.int32)
    alloc_check.check_tables(t, np.array([5, 12], np.int32), num_blocks=N, block_size=BS,
                             pad_value=PAD, shared=[3])


def test_free_count_and_slot_of():
    t, L = _valid_case()
    assert alloc_check.free_count(t, L, num_blocks=N, block_size=BS) == N - 5
    # position 6 of seq 0: logical block 1 (id 7), offset 2
    assert alloc_check.slot_of(t, 0, 6, BS) == 7 * BS + 2
    assert alloc_check.slot_of(t, 1, 0, BS) == 5 * BS


# ---- planted mistakes in the checker: each must let an invalid table through ----

def _mut_no_share_check(tables, lens, *, num_blocks, block_size, pad_value, shared=(), appended=True):
    # dropped the "held twice" rule entirely
    tables = np.asarray(tables)
    for i in range(len(lens)):
        nb = alloc_check.blocks_needed(lens[i], block_size)
        assert nb <= len(tables[i])
        for j in range(nb):
            assert 0 <= int(tables[i][j]) < num_blocks
        assert np.all(tables[i][nb:] == pad_value)


def _mut_full_rule_off_by_one(tables, lens, *, num_blocks, block_size, pad_value, shared=(), appended=True):
    # the shared block may hold the next write (<= L instead of <= L-1 for appended)
    return alloc_check.check_tables(tables, np.asarray(lens), num_blocks=num_blocks, block_size=block_size,
                                    pad_value=pad_value, shared=shared, appended=False) if appended else \
        alloc_check.check_tables(tables, np.asarray(lens) + 1, num_blocks=num_blocks, block_size=block_size,
                                 pad_value=pad_value, shared=shared, appended=False)


def _mut_no_padding_check(tables, lens, **kw):
    t = np.array(tables, copy=True)
    for i in range(len(lens)):
        t[i, alloc_check.blocks_needed(lens[i], kw["block_size"]):] = kw["pad_value"]
    return alloc_check.check_tables(t, lens, **kw)


def _mut_upper_bound_inclusive(tables, lens, **kw):
    kw = dict(kw)
    kw["num_blocks"] += 1
    return alloc_check.check_tables(tables, lens, **kw)


def _mut_any_index_shared(tables, lens, **kw):
    # shared blocks accepted at any logical index: relabel every shared use to index 0
    t = np.array(tables, copy=True)
    sh = set(int(x) for x in kw.get("shared", ()))
    out = []
    for i in range(len(lens)):
        row = [x for x in t[i] if int(x) in sh] + [x for x in t[i] if int(x) not in sh]
        out.append(row)
    return alloc_check.check_tables(np.array(out), lens, **kw)


CHECK_MUTANTS = {
    "no-share-check": _mut_no_share_check,
    "full-rule-off-by-one": _mut_full_rule_off_by_one,
    "no-padding-check": _mut_no_padding_check,
    "upper-bound-inclusive": _mut_upper_bound_inclusive,
    "shared-any-index": _mut_any_index_shared,
}


@pytest.mark.parametrize("name", sorted(CHECK_MUTANTS))
def test_checker_mutant_is_caught(name):
    mut = CHECK_MUTANTS[name]
    escaped = []
    for case, kw in _invalid_cases():
        try:
            _run(mut, kw)
            escaped.append(case)
        except AssertionError:
            pass
    assert escaped, f"checker mutant {name} still rejects every invalid table"


# ---- bits_to_f64 ----

FP16_POINTS = {
    0x3C00: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24, 0x0400: 2.0 ** -14,
    0x7BFF: 65504.0, 0x7C00: math.inf, 0xFC00: -math.inf, 0x3555: 0.333251953125, 0x0000: 0.0,
}
BF16_POINTS = {
    0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
    0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F80: math.inf, 0xFF80: -math.inf, 0x3EAB: 0.333984375,
    0x4049: 3.140625, 0x0000: 0.0,
}


def _decode_fields(bits, exp_bits, man_bits):
    """IEEE-style value of every pattern from its fields (independent of numpy's casts)."""
    bias = (1 << (exp_bits - 1)) - 1
    out = np.empty(bits.shape, np.float64)
    for i, b in enumerate(bits.tolist()):
        s = -1.0 if b >> (exp_bits + man_bits) else 1.0
        e = (b >> man_bits) & ((1 << exp_bits) - 1)
        m = b & ((1 << man_bits) - 1)
        if e == (1 << exp_bits) - 1:
            out[i] = s * math.inf if m == 0 else math.nan
        elif e == 0:
            out[i] = s * math.ldexp(m, 1 - bias - man_bits)
        else:
            out[i] = s * math.ldexp((1 << man_bits) + m, e - bias - man_bits)
    return out


def pin_fp16_points(f):
    for b, want in FP16_POINTS.items():
        got = f(np.array([b], np.uint16), "fp16")[0]
        assert got == want, (hex(b), got, want)
    nz = f(np.array([0x8000], np.uint16), "fp16")[0]
    assert nz == 0.0 and math.copysign(1.0, nz) < 0
    assert np.isnan(f(np.array([0x7E00, 0xFE01], np.uint16), "fp16")).all()


def pin_bf16_points(f):
    for b, want in BF16_POINTS.items():
        got = f(np.array([b], np.uint16), "bf16")[0]
        assert got == want, (hex(b), got, want)
    nz = f(np.array([0x8000], np.uint16), "bf16")[0]
    assert nz == 0.0 and math.copysign(1.0, nz) < 0
    assert np.isnan(f(np.array([0x7FC0, 0xFF81], np.uint16), "bf16")).all()


def pin_exhaustive(f):
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for dt, eb, mb in (("fp16", 5, 10), ("bf16", 8, 7)):
        got = f(allb, dt)
        want = _decode_fields(allb, eb, mb)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), dt
        assert np.array_equal(got[~nan], want[~nan]), dt
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), dt


BITS_PINS = [pin_fp16_points, pin_bf16_points, pin_exhaustive]


@pytest.mark.parametrize("pin", BITS_PINS, ids=[p.__name__ for p in BITS_PINS])
def test_bits_to_f64_pin(pin):
    pin(numerics.bits_to_f64)


def test_bits_to_f64_shape_and_dtype():
    x = np.array([[0x3C00, 0x4000]], np.uint16)
    got = numerics.bits_to_f64(x, "fp16")
    assert got.dtype == np.float64 and got.shape == (1, 2) and got.tolist() == [[1.0, 2.0]]
    with pytest.raises(ValueError):
        numerics.bits_to_f64(x, "fp32")


def _mut_fp16_astype(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.astype(np.float16).astype(np.float64)   # converts the integer's value
    return numerics.bits_to_f64(bits, dtype)


def _mut_bf16_shift8(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(8)).view(np.float32).astype(np.float64)
    return numerics.bits_to_f64(bits, dtype)


def _mut_sign_dropped(bits, dtype):
    return np.abs(numerics.bits_to_f64(bits, dtype))


def _mut_fp16_as_bf16(bits, dtype):
    return numerics.bits_to_f64(bits, "bf16")


BITS_MUTANTS = {
    "fp16-astype-instead-of-view": _mut_fp16_astype,
    "bf16-shift-8": _mut_bf16_shift8,
    "sign-dropped": _mut_sign_dropped,
    "fp16-read-as-bf16": _mut_fp16_as_bf16,
}


@pytest.mark.parametrize("name", sorted(BITS_MUTANTS))
def test_bits_mutant_is_caught(name):
    caught = []
    with np.errstate(all="ignore"):
        for pin in BITS_PINS:
            try:
                pin(BITS_MUTANTS[name])
            except (AssertionError, ValueError, OverflowError):
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
