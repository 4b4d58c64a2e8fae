"""Pins for the oracle's cache-byte and intensity formulas against figures the pages print."""

import math

import pytest

from oracle import cache_bytes as cb
from tests.conftest import read_tsv

UNITS = {"B": 1, "KiB": 2**10, "MiB": 2**20, "GiB": 2**30, "MB": 1e6, "GB": 1e9}

BYTE_ROWS = read_tsv("cache_bytes_printed.tsv")
RATIO_ROWS = read_tsv("ratios_printed.tsv")


@pytest.mark.parametrize("row", BYTE_ROWS, ids=[r[0] for r in BYTE_ROWS])
def test_printed_cache_bytes(row):
    _id, fname, args, exact, printed, unit, tol, _cite = row
    args = [int(a) for a in args.split(",")]
    got = getattr(cb, fname)(*args)
    assert got == int(exact)
    shown = got / UNITS[unit]
    assert abs(shown - float(printed)) <= float(tol) * float(printed) + 1e-12


def _ratio_value(rid):
    if rid == "p1_mla_vs_mha_per_layer":
        return cb.kv_bytes_per_token(1, 128, 128, 2) / cb.mla_bytes_per_token(1, 512, 64, 2)
    if rid == "p1_mla_gqa_head_equiv":
        return cb.mla_bytes_per_token(1, 512, 64, 2) / cb.kv_bytes_per_token(1, 1, 128, 2)
    if rid == "p2_s4_intensity_mha":
        return cb.decode_attention_intensity(64, 64, 2)
    if rid == "p2_s4_intensity_gqa8":
        return cb.decode_attention_intensity(64, 8, 2)
    if rid == "p2_s4_intensity_mqa_h64":
        return cb.decode_attention_intensity(64, 1, 2)
    if rid == "p2_s6_kv_size_gqa8":
        return cb.kv_bytes_per_token(80, 8, 128, 2) / cb.kv_bytes_per_token(80, 64, 128, 2)
    if rid == "p2_s6_kv_size_mla":
        return cb.mla_bytes_per_token(60, 512, 64, 2) / cb.kv_bytes_per_token(60, 128, 128, 2)
    if rid == "p2_s5_mla_vs_mha":
        return cb.kv_bytes_per_token(60, 128, 128, 2) / cb.mla_bytes_per_token(60, 512, 64, 2)
    if rid == "p2_s5_mla_vs_gqa8":
        return cb.kv_bytes_per_token(60, 16, 128, 2) / cb.mla_bytes_per_token(60, 512, 64, 2)
    if rid == "p3_first_step_removed":
        mha, gqa = cb.kv_bytes_per_token(32, 32, 128, 2), cb.kv_bytes_per_token(32, 8, 128, 2)
        return (mha - gqa) / mha
    if rid == "p3_second_step_removed":
        mha, gqa, mqa = (cb.kv_bytes_per_token(32, n, 128, 2) for n in (32, 8, 1))
        return (gqa - mqa) / mha
    raise KeyError(rid)


@pytest.mark.parametrize("row", RATIO_ROWS, ids=[r[0] for r in RATIO_ROWS])
def test_printed_ratios(row):
    rid, exact, printed, tol, _cite = row
    got = _ratio_value(rid)
    assert math.isclose(got, float(exact), rel_tol=1e-15)
    assert abs(got - float(printed)) <= float(tol) * float(printed) + 1e-15


def test_intensity_rises_with_group_size():
    # Exercise C of "MQA, GQA, and MLA" section 11: intensity scales with h/g.
    h = 64
    vals = [cb.decode_attention_intensity(h, g, 2) for g in (64, 32, 16, 8, 4, 2, 1)]
    assert vals == [1, 2, 4, 8, 16, 32, 64]
    # fp32 elements halve it; fp8 doubles it.
    assert cb.decode_attention_intensity(8, 2, 4) == 2
    assert cb.decode_attention_intensity(64, 8, 1) == 16


def test_intensity_independent_of_length_and_width():
    for S in (1, 512, 8192):
        for d in (64, 128, 576):
            assert cb.decode_attention_intensity(32, 8, 2, S, d) == 4


def test_whole_cache_is_per_token_times_tokens():
    for (nl, g, d, ctx, B, nb) in [(80, 8, 128, 8192, 32, 2), (32, 32, 128, 4096, 3, 1), (1, 1, 1, 1, 1, 4)]:
        assert cb.kv_cache_bytes(nl, g, d, ctx, B, nb) == cb.kv_bytes_per_token(nl, g, d, nb) * ctx * B
    assert cb.mla_cache_bytes(60, 512, 64, 8192, 3, 2) == cb.mla_bytes_per_token(60, 512, 64, 2) * 8192 * 3


def test_typescript_profiler_figures():
    # "Compressing the KV Cache ...", section "Profiling KV-Cache Memory in
    # TypeScript": the listing profiles 100 users at a 32768-token window and
    # prints MB = bytes / 2^20 and GB = bytes / 2^30 with two decimals.  The
    # page shows the code but not its output; the expected strings below are
    # worked by hand from the listing's arithmetic:
    #   LLaMA-3-70B: 2*80*8*128*32768*2 = 10 GiB per user -> "10240.00", x100 -> "1000.00"
    #   DeepSeek-V3: (512+64)*61*32768*2 = 2,302,672,896 B -> "2196.00", x100 -> "214.45"
    llama = cb.kv_cache_bytes(80, 8, 128, 32768, 1, 2)
    ds = cb.mla_cache_bytes(61, 512, 64, 32768, 1, 2)
    assert f"{llama / 2**20:.2f}" == "10240.00"
    assert f"{llama * 100 / 2**30:.2f}" == "1000.00"
    assert f"{ds / 2**20:.2f}" == "2196.00"
    assert f"{ds * 100 / 2**30:.2f}" == "214.45"


def test_llama2_4k_sequence_bytes():
    # "MQA, GQA, and MLA" section 1 prints "10.2 GB" per 4k sequence; the
    # exact size is 10 GiB = 10,737,418,240 B (the printed figure divides
    # 10,240 MiB by 1000).  ~49 concurrent sequences follow from
    # (640 - 140) GB of free memory over 10.24 GB per sequence.
    per_seq = cb.kv_cache_bytes(80, 64, 128, 4096, 1, 2)
    assert per_seq == 10 * 2**30
    assert math.floor((640 - 140) / (per_seq / 2**20 / 1000)) == 48
    assert round((640 - 140) / (per_seq / 2**20 / 1000)) == 49
