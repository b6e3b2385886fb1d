"""Every plausible mistake planted in the oracle must trip at least one pin.

Each mutant is a copy of oracle/kvc_oracle.c with one textual change (a
dropped term, a wrong sign or index, a transposed operand, a wrong head
mapping, an off-by-one in the mask or the append), compiled with gcc into a
temporary directory.  The pins are then run against the mutant in a child
process (a wrong index can write outside the test's arrays, which must not
corrupt this process); the test fails if all of them still pass.  The real
oracle is never modified.
"""
import json
import os
import shutil
import subprocess
import sys

import pytest

import oracle

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)

# Runs every pin against the library named on the command line and prints
# the names of the pins that tripped as one JSON line.
RUN_PINS = """
import json, sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
from oracle_pins import ALL_PINS
lib = oracle.load(sys.argv[1])
caught = []
for pin in ALL_PINS:
    try:
        pin(lib)
    except (AssertionError, oracle.OracleError, ValueError, FloatingPointError):
        caught.append(pin.__name__)
print(json.dumps(caught), flush=True)
""".format(root=ROOT, tests=TESTS)

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
                             "load_elem(k_cache, cache_row(layer, b, hkv, d % n, B, Hkv, Tmax, D) + j % D, dtype);"),
    # the softmax
    "exp_sign_flipped": ("const double w = exp(s[j] - m);", "const double w = exp(m - s[j]);"),
    "no_normalisation": ("out_row[d] = acc[d] / denom;", "out_row[d] = acc[d];"),
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
    # packed variable-length prefill: token offsets, history offset, head
    "varlen_mask_without_history": ("hist_len[b] + i + 1, scale, s, acc, out + qrow);",
                                    "i + 1, scale, s, acc, out + qrow);"),
    "varlen_append_at_position_i": ("const int pos = hist_len[b] + i;", "const int pos = i;"),
    "varlen_query_head_major": ("const size_t qrow = (((size_t)l * T + cu_seqlens[b] + i) * Hq + hq) * (size_t)D;",
                                "const size_t qrow = (((size_t)l * Hq + hq) * T + cu_seqlens[b] + i) * (size_t)D;"),
    "varlen_tokens_head_major": ("const size_t src = (((size_t)l * T + cu_seqlens[b] + i) * Hkv + h) * (size_t)D;",
                                 "const size_t src = (((size_t)l * Hkv + h) * T + cu_seqlens[b] + i) * (size_t)D;"),
    "paged_prefill_writes_history_slots": ("for (int npos = hist_len[b]; npos < hist_len[b] + cu_seqlens[b + 1] - cu_seqlens[b]; ++npos) {",
                                           "for (int npos = 0; npos < cu_seqlens[b + 1] - cu_seqlens[b]; ++npos) {"),
    # the paged cache: block-table lookup, row inside the block, head, layer
    "paged_append_block_from_offset": ("block_table[(size_t)b * max_blocks + t / block_size]",
                                       "block_table[(size_t)b * max_blocks + t % block_size]"),
    "paged_append_row_from_block_index": ("paged_row(layer0 + l, blk, h, t % block_size,",
                                          "paged_row(layer0 + l, blk, h, t / block_size % block_size,"),
    "paged_gather_row_off_by_one": ("paged_row(layer0 + l, blk, h, pos % block_size,",
                                    "paged_row(layer0 + l, blk, h, (pos + 1) % block_size,"),
    "paged_gather_ignores_layer0": ("paged_row(layer0 + l, blk, h, pos % block_size,",
                                    "paged_row(l, blk, h, pos % block_size,"),
    "paged_table_row_of_first_sequence": ("block_table[(size_t)b * max_blocks + pos / block_size]",
                                          "block_table[pos / block_size]"),
    "paged_ignores_head": ("((((size_t)l * num_blocks + blk) * Hkv + h)",
                           "((((size_t)l * num_blocks + blk) * Hkv + 0)"),
    "paged_head_and_row_swapped": ("((((size_t)l * num_blocks + blk) * Hkv + h) * (size_t)block_size +\n          (size_t)r)",
                                   "((((size_t)l * num_blocks + blk) * (size_t)block_size + r) * Hkv +\n          (size_t)h)"),
    "paged_capacity_unchecked": ("if (end > (int64_t)max_blocks * block_size) return ORACLE_E_CAPACITY;",
                                 "if (end > (int64_t)max_blocks * block_size + block_size) return ORACLE_E_CAPACITY;"),
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
    r = subprocess.run([sys.executable, "-c", RUN_PINS, so], capture_output=True, text=True,
                       timeout=600, env=dict(os.environ, OMP_NUM_THREADS="2"))
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("[")]
    if lines:
        caught = json.loads(lines[-1])
    else:
        # the mutant crashed the child before the pins finished: a visible
        # failure no correct oracle shows, so the mistake did not go unnoticed
        assert r.returncode != 0, r.stderr[-2000:]
        caught = [f"crash ({r.returncode})"]
    assert caught, f"planted mistake {name!r} passed every pin"
