"""Planted mistakes in the oracle must fail at least one pin.

Each case copies ``oracle/attn.c``, applies one textual mutation (a dropped
term, a wrong index, a transposed layout, a wrong sign...), compiles it with
gcc into a temporary library, swaps it in for the real oracle and runs every
pin.  The real oracle is restored afterwards.  CPU only.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as orc_build

SRC = os.path.join(os.path.dirname(orc_build.LIB), "attn.c")

MUTANTS = {
    "scale_dropped": ("s[j] = scale * acc;", "s[j] = acc;"),
    "no_normalisation": ("o[d] /= l;", "o[d] /= 1.0;"),
    "block_index_mod": ("max_blocks + j / BLOCK]", "max_blocks + j % BLOCK]"),
    "slot_offset_div": ("j % BLOCK, d", "j / BLOCK, d"),
    "gqa_map_modulo": ("g = h / G;", "g = h % Hkv;"),
    "k_layout_chunk_swapped": ("(size_t)(d / X)) * BLOCK + (size_t)t) * X + (size_t)(d % X)",
                               "(size_t)(d % X)) * BLOCK + (size_t)t) * X + (size_t)(d / X)"),
    "v_layout_transposed": ("(size_t)D + (size_t)d) * BLOCK + (size_t)t",
                            "(size_t)BLOCK + (size_t)t) * D + (size_t)d"),
    "merge_sign": ("L += pl[p] * exp(pm[p] - M);", "L += pl[p] * exp(M - pm[p]);"),
    "merge_drop_rescale": ("o[d] += po[(size_t)p * D + d] * f;", "o[d] += po[(size_t)p * D + d];"),
    "bf16_widen_shift": ("<< 16;", "<< 15;"),
    "query_row_of_head0": ("elem(q, (size_t)bh * D + d, qt)", "elem(q, (size_t)b * Hq * D + d, qt)"),
    "context_off_by_one": ("int n = ctx[b];", "int n = ctx[b] - 1;"),
    "append_skips_slot0": ("if (s < 0) continue;", "if (s <= 0) continue;"),
    "copy_only_k": ("copy_elem(vpool, v_at(dst,", "if (0) copy_elem(vpool, v_at(dst,"),
    "value_of_next_token": ("w * vval(vpool, blk, g, j % BLOCK, d",
                            "w * vval(vpool, blk, g, (j + 1) % BLOCK, d"),
    "max_from_first_token_only": ("if (s[j] > m) m = s[j];", "if (j == 0) m = s[j];"),
    "int8_scale_dropped": ("return v * (double)sc;", "return v;"),
    "int8_truncating_round": ("float r = rintf(v / scale);", "float r = truncf(v / scale);"),
    "int8_signed_amax": ("float a = fabsf(v);", "float a = v;"),
    "int8_scale_of_next_slot": ("memcpy(&sc, tile + (size_t)16 * D + 4 * (size_t)t, sizeof sc);",
                                "memcpy(&sc, tile + (size_t)16 * D + 4 * (size_t)((t + 1) % BLOCK), sizeof sc);"),
    "int8_v_read_as_k": ("size_t at = is_v ? (size_t)d * BLOCK + t : ((size_t)(d / 16)",
                         "size_t at = !is_v ? (size_t)d * BLOCK + t : ((size_t)(d / 16)"),
    "int8_scale_255": ("? 448.0f : 127.0f", "? 448.0f : 255.0f"),
    "fp8_scale_127": ("? 448.0f : 127.0f", "? 127.0f : 127.0f"),
    "fp8_read_as_int8": ("double v = dtype == 3 ? e4m3_value", "double v = dtype == 4 ? e4m3_value"),
    "fp8_decode_bias_8": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "fp8_decode_no_subnormals": ("ldexp(m / 8.0, -6)", "ldexp(1.0 + m / 8.0, -7)"),
    "fp8_decode_sign_dropped": ("return (c & 0x80) ? -v : v;", "return v;"),
    "fp8_encode_bias_8": ("int E = e - 1 + 7;", "int E = e - 1 + 8;"),
    "fp8_encode_ties_away": ("double q = nearbyint((2.0 * f - 1.0) * 8.0);", "double q = round((2.0 * f - 1.0) * 8.0);"),
    "fp8_encode_truncates": ("double q = nearbyint((2.0 * f - 1.0) * 8.0);", "double q = floor((2.0 * f - 1.0) * 8.0);"),
    "fp8_encode_no_carry": ("if (q == 8.0) {", "if (q == 9.0) {"),
    "fp8_encode_subnormal_flush": ("return s | (unsigned char)nearbyint(a * 512.0);", "return s;"),
    "fp8_encode_sign_dropped": ("unsigned char s = signbit(y) ? 0x80 : 0;", "unsigned char s = 0;"),
    "fp8_saturate_to_nan": ("if (a >= 448.0) return s | 0x7E;", "if (a >= 448.0) return s | 0x7F;"),
    "prefill_causal_exclusive": ("int n = ctx[b] - nq + t + 1;", "int n = ctx[b] - nq + t;"),
    "prefill_without_prefix": ("int n = ctx[b] - nq + t + 1;", "int n = t + 1;"),
    "prefill_whole_context": ("int n = ctx[b] - nq + t + 1;", "int n = ctx[b];"),
    "prefill_query_of_first_token": ("elem(q, (size_t)rh * D + d, qt)", "elem(q, ((size_t)qstart[b] * Hq + h) * D + d, qt)"),
    "int8_copy_k_only": ("memcpy((char *)vpool + dst * tb", "if (0) memcpy((char *)vpool + dst * tb"),
    "int8_k_slots_in_plain_order": ("return (size_t)((t & 3) | ((t & 4) << 1) | ((t & 8) >> 1));", "return (size_t)t;"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC, encoding="utf-8").read()
    assert old in src, f"mutation {name} does not apply"
    out = tmp_path / f"attn_{name}.c"
    out.write_text(src.replace(old, new), encoding="utf-8")
    lib = tmp_path / f"liborc_{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(lib), str(out), "-lm"], check=True)
    return str(lib)


_RUNNER = r"""
import ctypes, sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
import pins
from oracle import attn as orc
real = orc.lib()
mutant = ctypes.CDLL(sys.argv[1])
for fn in ("orc_append", "orc_copy_blocks", "orc_paged_attention", "orc_contiguous_attention",
           "orc_partitioned_attention", "orc_gather_token", "orc_num_threads", "orc_paged_prefill"):
    getattr(mutant, fn).argtypes = getattr(real, fn).argtypes
    getattr(mutant, fn).restype = getattr(real, fn).restype
orc._lib = mutant
for check in pins.ALL_CHECKS:
    print("RUN", check.__name__, flush=True)
    try:
        check()
    except Exception as e:
        print("FAILED", check.__name__, type(e).__name__, flush=True)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    """Runs the pins in a child process: an out-of-bounds mutant may crash it,
    which also counts as caught."""
    old, new = MUTANTS[name]
    path = _build_mutant(tmp_path, name, old, new)
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(tests_dir)
    r = subprocess.run([sys.executable, "-c", _RUNNER, path, tests_dir, root],
                       capture_output=True, text=True, timeout=300)
    assert "RUN check_brute_force" in r.stdout, r.stderr
    failed = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
    crashed = r.returncode < 0  # killed by a signal inside a check
    assert r.returncode <= 0, r.stderr
    assert failed or crashed, f"no pin caught mutation {name}:\n{r.stdout}\n{r.stderr}"
