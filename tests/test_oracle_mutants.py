"""Planted mistakes in the CPU oracle must be caught by its pins.

Each mutant is a copy of ``oracle/ep_oracle.c`` with one plausible mistake (a
dropped term, a wrong index, a reversed order, a wrong rounding), compiled
with gcc into a temporary directory.  The pin suite (``tests/pins.py``) is run
against it in a subprocess; at least one pin must fail.  Nothing here touches
a GPU.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

SRC = os.path.join(ROOT, "oracle", "ep_oracle.c")

MUTANTS = {
    "no_alignment": ("int64_t aligned = (counts[e] + A - 1) / A * A;",
                     "int64_t aligned = counts[e];"),
    "reverse_segment_order": ("int32_t row = psum[e] + fill[e];",
                              "int32_t row = psum[e] + counts[e] - 1 - fill[e];"),
    "invalid_not_counted": ("                ++invalid;\n", "\n"),
    "recv_counts_slots": ("        num_recv += any;", "        num_recv += K;"),
    "gap_meta_zero": ("            src_meta[r] = -1;", "            src_meta[r] = 0;"),
    "capacity_check_loose": ("if (run > capacity)", "if (run > capacity + A)"),
    "bound_ignores_min": ("int64_t per_token = K < E ? K : E;", "int64_t per_token = K;"),
    "bound_not_rounded": ("return (n + A - 1) / A * A;", "return n;"),
    "dispatch_wrong_token": ("x + t * row_bytes, (size_t)row_bytes);",
                             "x + ((t + 1) % T) * row_bytes, (size_t)row_bytes);"),
    "dispatch_sf_strides_swapped": ("sf[t * sf_ts + j * sf_hs]", "sf[t * sf_hs + j * sf_ts]"),
    "dispatch_gap_sf_kept": ("                out_sf[r * o_ts + j * o_hs] = 0;\n", "\n"),
    "dispatch_weight_index": ("out_w[r] = w ? w[t * K + k] : 1.0f;",
                              "out_w[r] = w ? w[t * K] : 1.0f;"),
    "dispatch_pads_no_weight": ("                out_w[r] = 0.0f;\n", "                ;\n"),
    "combine_no_bias": ("v = v + bf16_to_f32(bias[e * H + h]);", "v = v;"),
    "combine_bias_wrong_expert": ("int64_t e = topk_idx[t * K + k];\n                    v = v",
                                  "int64_t e = k % 1;\n                    v = v"),
    "combine_bias_after_weight": (
        "float p = w ? w[t * K + k] * v : v;",
        "float p = w ? w[t * K + k] * bf16_to_f32(y[r * H + h]) + (v - bf16_to_f32(y[r * H + h])) : v;"),
    "combine_no_weight": ("float p = w ? w[t * K + k] * v : v;", "float p = v;"),
    "combine_truncate": ("u += 0x7FFFu + lsb;", "u += 0u * lsb;"),
    "combine_round_half_up": ("u += 0x7FFFu + lsb;", "u += 0x8000u + 0u * lsb;"),
    "combine_double_accumulator": ("            float acc = 0.0f;\n            for (int64_t k = 0; k < K; ++k) {\n                int64_t r = dst[t * K + k];\n                if (r < 0)\n                    continue;\n                float v",
                                   "            double acc = 0.0;\n            for (int64_t k = 0; k < K; ++k) {\n                int64_t r = dst[t * K + k];\n                if (r < 0)\n                    continue;\n                float v"),
    "combine_reverse_k": ("            float acc = 0.0f;\n            for (int64_t k = 0; k < K; ++k) {",
                          "            float acc = 0.0f;\n            for (int64_t k = K - 1; k >= 0; --k) {"),
    "combine_fused_multiply_add": ("                float p = w ? w[t * K + k] * v : v;\n                acc = acc + p;",
                                   "                float p = w ? w[t * K + k] * v : v;\n                acc = w ? __builtin_fmaf(w[t * K + k], v, acc) : acc + p;"),
    "combine_neg_zero_start": ("float acc = 0.0f;\n            for (int64_t k = 0; k < K; ++k) {\n                int64_t r = dst[t * K + k];\n                if (r < 0)\n                    continue;\n                float v",
                               "float acc = -0.0f;\n            for (int64_t k = 0; k < K; ++k) {\n                int64_t r = dst[t * K + k];\n                if (r < 0)\n                    continue;\n                float v"),
    "cb_grad_y_no_weight": ("float s = w ? w[t * K + k] * gv : gv;", "float s = gv;"),
    "cb_grad_w_no_bias": ("v += (double)bf16_to_f32(bias[e * H + h]);", "v += 0.0;"),
    "cb_grad_w_wrong_row": (
        "if (grad_w) {\n                    double v = (double)bf16_to_f32(y[r * H + h]);",
        "if (grad_w) {\n                    double v = (double)bf16_to_f32(y[(r > 0 ? r - 1 : r) * H + h]);"),
    "cb_grad_w_no_grad": ("acc += (double)gv * v;", "acc += v;"),
    "cb_grad_bias_skips_last_row": (
        "for (int64_t r = psum[e]; r < (int64_t)psum[e] + counts[e]; ++r) {",
        "for (int64_t r = psum[e]; r < (int64_t)psum[e] + counts[e] - 1; ++r) {"),
    "cb_grad_bias_no_weight": ("acc += w ? (double)w[i] * gv : gv;", "acc += gv;"),
    "db_grad_w_wrong_row": ("grad_w[i] = (dst[i] >= 0 && gw) ? gw[dst[i]] : 0.0f;",
                            "grad_w[i] = (dst[i] >= 0 && gw) ? gw[i % 7] : 0.0f;"),
    "rank_counts_invalid_ids": ("            if (e >= 0 && e < E)\n                any = 1;",
                                "            if (e != -1)\n                any = 1;"),
    "rank_row_off_by_one": ("recv_row[t] = (int32_t)rows;", "recv_row[t] = (int32_t)rows + (t > 2);"),
    "rank_idx_not_masked": ("out_idx[r * K + k] = valid ? e : -1;", "out_idx[r * K + k] = e;"),
    "rank_weight_kept_on_empty": ("out_w[r * K + k] = valid ? (w ? w[t * K + k] : 1.0f) : 0.0f;",
                                  "out_w[r * K + k] = w ? w[t * K + k] : 1.0f;"),
    "rank_combine_b1_first": (
        "            float acc = r >= 0 ? bf16_to_f32(x[r * H + h]) : 0.0f;\n"
        "            if (b0)\n                acc = acc + bf16_to_f32(b0[t * H + h]);\n"
        "            if (b1)\n                acc = acc + bf16_to_f32(b1[t * H + h]);",
        "            float acc = r >= 0 ? bf16_to_f32(x[r * H + h]) : 0.0f;\n"
        "            if (b1)\n                acc = acc + bf16_to_f32(b1[t * H + h]);\n"
        "            if (b0)\n                acc = acc + bf16_to_f32(b0[t * H + h]);"),
    "token_bias_before_slots": ('            float acc = 0.0f;\n            for (int64_t k = 0; k < K; ++k) {\n                int64_t r = dst[t * K + k];\n                if (r < 0)\n                    continue;\n                float v = bf16_to_f32(y[r * H + h]);\n                if (bias) {\n                    int64_t e = topk_idx[t * K + k];\n                    v = v + bf16_to_f32(bias[e * H + h]);\n                }\n                float p = w ? w[t * K + k] * v : v;\n                acc = acc + p;\n            }\n            if (b0)\n                acc = acc + bf16_to_f32(b0[t * H + h]);',
        '            float acc = b0 ? bf16_to_f32(b0[t * H + h]) : 0.0f;\n            for (int64_t k = 0; k < K; ++k) {\n                int64_t r = dst[t * K + k];\n                if (r < 0)\n                    continue;\n                float v = bf16_to_f32(y[r * H + h]);\n                if (bias) {\n                    int64_t e = topk_idx[t * K + k];\n                    v = v + bf16_to_f32(bias[e * H + h]);\n                }\n                float p = w ? w[t * K + k] * v : v;\n                acc = acc + p;\n            }\n'),
    "token_bias_b1_dropped": (
        "                acc = acc + p;\n            }\n            if (b0)\n"
        "                acc = acc + bf16_to_f32(b0[t * H + h]);\n            if (b1)\n"
        "                acc = acc + bf16_to_f32(b1[t * H + h]);",
        "                acc = acc + p;\n            }\n            if (b0)\n"
        "                acc = acc + bf16_to_f32(b0[t * H + h]);\n            if (0)\n"
        "                acc = acc + bf16_to_f32(b1[t * H + h]);"),
    "quant_ties_up": ("if (dhi < dlo || (dhi == dlo && ((lo + 1) & 1) == 0))",
                      "if (dhi < dlo || dhi == dlo)"),
    "quant_no_scale_floor": ("float s = (amax > 1e-12f ? amax : 1e-12f) / 448.0f;",
                             "float s = amax / 448.0f;"),
    "quant_ue8m0_rounds_down": ("                    ++e;                  /* round up", 
                                "                    e += 0;               /* round up"),
    "quant_pack_order": ("|= e << (8 * (j % 4));", "|= e << (8 * (3 - j % 4));"),
    "quant_signed_amax": ("& 0x7FFFFFFFu);\n                if (a > amax)",
                          "& 0xFFFFFFFFu);\n                if (a > amax)"),
    "quant_nan_code": ("    if (v != v)\n        return 0x7F;", "    if (v != v)\n        return 0x00;"),
    "quant_subnormal_step": ("return e == 0 ? m * pow2(-9)", "return e == 0 ? m * pow2(-10)"),
    "quant_ue8m0_divides_by_s": ("divisor = bits_f32(e << 23);", "divisor = s;"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


def test_unmutated_oracle_passes_every_pin(tmp_path):
    so = str(tmp_path / "lib_clean.so")
    oracle.build(SRC, so)
    out = subprocess.run([sys.executable, "-m", "tests.pins", so], cwd=ROOT,
                         capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    res = json.loads(out.stdout.strip().splitlines()[-1])
    assert all(v is None for v in res.values()), res


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"anchor for {name} is not unique"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(old, new))
    so = str(tmp_path / f"{name}.so")
    oracle.build(str(src), so, extra=["-w"])
    out = subprocess.run([sys.executable, "-m", "tests.pins", so], cwd=ROOT,
                         capture_output=True, text=True, timeout=300)
    if out.returncode != 0:          # the mutant crashed the pin run: caught
        return
    res = json.loads(out.stdout.strip().splitlines()[-1])
    failed = [k for k, v in res.items() if v is not None]
    assert failed, f"mutant {name} passed every pin"
