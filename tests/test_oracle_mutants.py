"""Every plausible mistake planted in the oracle must trip at least one pin.

Each mutant is a copy of oracle/kvc_oracle.c with one textual change (a
dropped term, a wrong sign or index, a transposed operand, a wrong head
mapping, an off-by-one in the mask or the append), compiled with gcc into a
temporary directory.  The pins are then run against the mutant; the test
fails if all of them still pass.  The real oracle is never modified.
"""
import os
import shutil

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "kvc_oracle.c")

MUTANTS = {
    # the mask: P+i+1 visible keys
    "mask_one_short": ("const int n = hist_len[b] + i + 1;", "const int n = hist_len[b] + i + (i > 0);"),
    "mask_without_row_offset": ("const int n = hist_len[b] + i + 1;", "const int n = hist_len[b] + N;"),
    "mask_without_history_offset": ("const int n = hist_len[b] + i + 1;", "const int n = i + 1;"),
    # GQA head mapping
    "gqa_interleaved": ("const int hkv = hq / group;", "const int hkv = hq % Hkv;"),
    # the score
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "scale_inverted": ("s[j] = scale * dot;", "s[j] = dot / scale;"),
    "scores_from_values": ("load_elem(k_cache, krow + d, dtype);", "load_elem(v_cache, krow + d, dtype);"),
    "key_index_transposed": ("load_elem(k_cache, krow + d, dtype);",
                             "load_elem(k_cache, cache_row(layer0 + l, b, hkv, d % n, B, Hkv, Tmax, D) + j % D, dtype);"),
    # the softmax
    "exp_sign_flipped": ("const double w = exp(s[j] - m);", "const double w = exp(m - s[j]);"),
    "no_normalisation": ("out[qrow + d] = acc[d] / denom;", "out[qrow + d] = acc[d];"),
    "denominator_counts_keys": ("denom += w;", "denom += 1.0;"),
    "weights_not_applied": ("acc[d] += w * load_elem(v_cache, vrow + d, dtype);",
                            "acc[d] += load_elem(v_cache, vrow + d, dtype) / n;"),
    # the append
    "append_one_slot_late": ("size_t dst = cache_row(layer0 + l, b, h, hist_len[b] + i, B, Hkv,",
                             "size_t dst = cache_row(layer0 + l, b, h, hist_len[b] + i + (i + 1 < N), B, Hkv,"),
    "append_ignores_layer0": ("size_t dst = cache_row(layer0 + l, b, h, hist_len[b] + i, B, Hkv,",
                              "size_t dst = cache_row(l, b, h, hist_len[b] + i, B, Hkv,"),
    "append_values_from_keys": ("memcpy((char *)v_cache + dst * es, (const char *)v_new + src * es,",
                                "memcpy((char *)v_cache + dst * es, (const char *)k_new + src * es,"),
    # element decoding
    "bf16_wrong_shift": ("uint32_t bits = (uint32_t)hi << 16;", "uint32_t bits = (uint32_t)hi << 15;"),
    # the size formula
    "size_formula_drops_kv_factor": ("return (uint64_t)(2 * layers *", "return (uint64_t)(1 * layers *"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique in the oracle"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    oracle.compile_library(str(src), so)
    lib = oracle.load(so)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, oracle.OracleError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
