"""Each planted mistake in a copy of the oracle must fail at least one pin.

The mistakes are the plausible ones: a flipped sign, a wrong index, a dropped term,
a transposed operand, a wrong rounding. Each mutant is compiled from a text-edited
copy of oracle/kvq_oracle.cpp into a temporary directory and the pins of
tests/oracle_pins.py run against it in a child process (so a mutant that crashes
also counts as caught). Nothing here touches the real oracle build or a GPU.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvq_oracle.cpp")

# (name, original text, replacement)
MUTANTS = [
    ("butterfly_sign", "x[i + h] = a - b;", "x[i + h] = b - a;"),
    ("hadamard_or", "popcount_u32((uint32_t)(i & j))", "popcount_u32((uint32_t)(i | j))"),
    ("rotation_const", "return ldexpf(sqrtf(2.0f), -(k + 1) / 2);", "return ldexpf(sqrtf(2.0f), -(k - 1) / 2);"),
    ("dense_rot_no_scale", "y[b + i] = acc * inv;", "y[b + i] = acc;"),
    ("zero_from_max", "orc_f32_to_f16(mn + 0.0f)", "orc_f32_to_f16(mx + 0.0f)"),
    ("scale_by_2pow", "float s32 = range / (float)qmax;", "float s32 = range / (float)(qmax + 1);"),
    ("minmax_scan_short", "for (int i = 1; i < group; ++i) {", "for (int i = 1; i < group - 1; ++i) {"),
    ("floor_not_rint", "float r = rintf(u);", "float r = floorf(u);"),
    ("no_lower_clamp", "if (r < 0.0f) c = 0;", ""),
    ("nibble_order",
     "packed[k / per_byte] |= (uint8_t)(codes[k] << (bits * (k % per_byte)));",
     "packed[k / per_byte] |= (uint8_t)(codes[k] << (bits * (per_byte - 1 - k % per_byte)));"),
    ("f16_ties_down", "if (rem > half || (rem == half && (whole & 1u))) whole += 1;", "if (rem > half) whole += 1;"),
    ("dequant_no_zero", "out[i] = fmaf((float)codes[i], s, z);", "out[i] = fmaf((float)codes[i], s, 0.0f);"),
    ("v_rotated_too", "if (which == 0) orc_rotate(x, d, c->hadamard_block); /* keys only */",
     "orc_rotate(x, d, c->hadamard_block);"),
    ("gqa_modulo", "int h = j / ratio;\n      double* o = out + ((int64_t)b * num_q_heads + j) * d;\n      if (T <= 0)",
     "int h = j % c->num_kv_heads;\n      double* o = out + ((int64_t)b * num_q_heads + j) * d;\n      if (T <= 0)"),
    ("softmax_scale", "double sigma = softmax_scale > 0.0 ? softmax_scale : 1.0 / sqrt((double)d);\n  double* qv",
     "double sigma = softmax_scale > 0.0 ? softmax_scale : 1.0 / (double)d;\n  double* qv"),
    ("v_tokens_not_interleaved", "return base + tile + (int64_t)w * 32 + (o / 2) * 4 + b * 2 + (o % 2);",
     "return base + tile + (int64_t)w * 32 + o * 2 + b;"),
    ("k_tile_token_major", "return base + tile + ((int64_t)(k / 16) * 16 + o) * 16 + k % 16;",
     "return base + tile + (int64_t)o * row_bytes(c) + k;"),
    ("v_meta_parts_swapped", "(((int64_t)part * n_groups(c) + g) * 2 + half) * 4 + i) * 4;",
     "(((int64_t)half * n_groups(c) + g) * 2 + part) * 4 + i) * 4;"),
    ("window_evict_late", "if (!w->residual && t >= S && t - R >= S) quantize_store_pair(c, kw, vw, evict_slots[r], h);",
     "if (!w->residual && t >= S && t - R > S) quantize_store_pair(c, kw, vw, evict_slots[r], h);"),
    ("window_ring_index", "return t < w->sink ? t : w->sink + (t - w->sink) % w->recent;",
     "return t < w->sink ? t : w->sink + (t - w->sink + 1) % w->recent;"),
    ("window_recent_edge", "return t < w->sink || t >= T - w->recent;", "return t < w->sink || t > T - w->recent;"),
    ("window_query_rotated", "for (int i = 0; i < d; ++i) dot += qv[i] * (double)orc_bf16_to_f32(kw[i]);",
     "for (int i = 0; i < d; ++i) dot += qr[i] * (double)orc_bf16_to_f32(kw[i]);"),
    ("meta_swapped", "      put_u16(m, scale[g]);\n      put_u16(m + 2, zero[g]);\n    }\n  } else {",
     "      put_u16(m, zero[g]);\n      put_u16(m + 2, scale[g]);\n    }\n  } else {"),
    ("q_not_rotated", "orc_rotate_dense_f64(qv, qr, d, c->hadamard_block);", "orc_rotate_dense_f64(qv, qr, d, 0);"),
    ("softmax_no_norm", "for (int i = 0; i < d; ++i) o[i] = acc[i] / den;", "for (int i = 0; i < d; ++i) o[i] = acc[i];"),
    ("hybrid_tie_to_symmetric", "if (err_s < err_a) {", "if (err_s <= err_a) {"),
    ("hybrid_choice_inverted", "if (err_s < err_a) {", "if (err_s > err_a) {"),
    ("hybrid_sym_divisor", "a / (float)(mid - 1)", "a / (float)mid"),
    ("hybrid_sym_zero_sign", "-((float)mid * orc_f16_to_f32(ss16)) + 0.0f", "((float)mid * orc_f16_to_f32(ss16)) + 0.0f"),
    ("hybrid_ignored_in_cache", "c->quant_mode == 1, codes, sc, ze", "0, codes, sc, ze"),
    ("prune_chunk_width", "int width = 128 / c->bits; /* channels of one 16-byte chunk",
     "int width = 64 / c->bits; /* channels of one 16-byte chunk"),
    ("prune_bit_order", "if (!((mask >> (i / width)) & 1)) qr[i] = 0.0;", "if (!((mask >> (d / width - 1 - i / width)) & 1)) qr[i] = 0.0;"),
    ("prune_mask_ignored", "if (!((mask >> (i / width)) & 1)) qr[i] = 0.0;", "(void)mask;"),
    ("prune_energy_abs", "+= qr[i] * qr[i];", "+= fabs(qr[i]);"),
    ("vt_entry_bits_swapped", "t = 4 * (ch / 64) + 2 * (ch % 2) + (ch % 4) / 2;", "t = 4 * (ch / 64) + (ch % 2) + 2 * ((ch % 4) / 2);"),
    ("vt_groups_along_channels", "      quantize_store_token_group(c, k_new + r * stride, v_new + r * stride, slots + r, stride, stride);",
     "      for (int i = 0; i < G; ++i) for (int h = 0; h < c->num_kv_heads; ++h) quantize_store_pair(c, k_new + (r + i) * stride + h * d, v_new + (r + i) * stride + h * d, slots[r + i], h);"),
    ("vt_meta_wrong_group", "c->v_meta + vt_meta_off(c, page, h, off / c->group_size, i);", "c->v_meta + vt_meta_off(c, page, h, 0, i);"),
    ("residual_whole_ring", "if (w->residual) return t >= T - T % w->recent;", "if (w->residual) return t >= T - w->recent;"),
    ("residual_group_early", "if (w->residual && (t + 1) % R == 0) {", "if (w->residual && t % R == 0) {"),
]

RUNNER = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, oracle_pins as pins
with oracle.using({lib!r}):
    for chk in pins.ALL_CHECKS + [lambda: pins.check_f16_conversion_f16c(full=False)]:
        try:
            chk()
        except AssertionError:
            print("CAUGHT", getattr(chk, "__name__", "f16c")); sys.exit(0)
print("SURVIVED"); sys.exit(0)
"""


def _run(name, old, new, tmp):
    src = open(SRC).read()
    # a pattern shared by the plain and the windowed decode is mutated in both
    assert src.count(old) >= 1, f"mutant {name}: pattern not found"
    path = os.path.join(tmp, f"mut_{name}.cpp")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    # the mutant includes the oracle's header from the source tree
    lib = oracle.build(path, os.path.join(tmp, f"libmut_{name}.so"), extra=[f"-I{os.path.dirname(SRC)}"])
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    out = r.stdout.strip().splitlines()
    if r.returncode != 0:
        return name, f"CAUGHT (crashed: rc={r.returncode})"
    return name, out[-1] if out else "NO OUTPUT"


def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            results = list(ex.map(lambda m: _run(*m, tmp), MUTANTS))
    survived = [n for n, r in results if not r.startswith("CAUGHT")]
    assert not survived, f"mutants not caught by any pin: {survived}; all: {results}"
