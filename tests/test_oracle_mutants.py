"""The pins catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of moe_oracle.c (on the CPU, in a
temporary directory), builds it, and replays every pin against it: at least one
pin must fail. This shows the pins constrain each part of the oracle: the
placement of experts on ranks, the per-rank dedupe, the scan offsets, the
token order, the permute's rank test and bookkeeping, the combine's slots,
weights and rounding.
"""
import os
import subprocess
import sys

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")
TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)

MUTANTS = {
    "round-robin placement": (
        "on_rank[e / m] = 1;\n    }\n    for (int32_t r = 0; r < R; ++r) rank_counts[r] += on_rank[r];",
        "on_rank[e % R] = 1;\n    }\n    for (int32_t r = 0; r < R; ++r) rank_counts[r] += on_rank[r];"),
    "one copy per expert": (
        "      expert_counts[e] += 1;\n      on_rank[e / m] = 1;",
        "      expert_counts[e] += 1;\n      on_rank[e / m] += 1;"),
    "inclusive rank scan": (
        "for (int32_t r = 0; r < R; ++r) next_rank[r] = rank_offsets[r];",
        "for (int32_t r = 0; r < R; ++r) next_rank[r] = rank_offsets[r + 1];"),
    "expert runs start one late": (
        "for (int32_t e = 0; e < E; ++e) next_expert[e] = expert_offsets[e];",
        "for (int32_t e = 0; e < E; ++e) next_expert[e] = expert_offsets[e] + (e > 0);"),
    "tokens walked backwards": (
        "  for (int32_t t = 0; t < T; ++t) {\n    memset(on_rank, 0, (size_t)R);\n    for (int32_t j = 0; j < k; ++j) {\n      const int32_t e = topk_ids[(int64_t)t * k + j];\n      if (!id_is_expert(e, E)) {\n        pair_row",
        "  for (int32_t t = T - 1; t >= 0; --t) {\n    memset(on_rank, 0, (size_t)R);\n    for (int32_t j = 0; j < k; ++j) {\n      const int32_t e = topk_ids[(int64_t)t * k + j];\n      if (!id_is_expert(e, E)) {\n        pair_row"),
    "-1 reported as bad": (
        "if (e != -1) err |= ORACLE_ERR_BAD_ID;",
        "err |= ORACLE_ERR_BAD_ID;"),
    "pack records wrong token": (
        "rank_src_token[row] = t;",
        "rank_src_token[row] = t + (r > 0);"),
    "permute wrong rank test": (
        "if (!id_is_expert(e, E) || e / m != r) continue;\n      const int64_t dst",
        "if (!id_is_expert(e, E)) continue;\n      const int64_t dst"),
    "permute wrong pair id": (
        "expert_src_pair[dst] = t * k + j;",
        "expert_src_pair[dst] = t * k;"),
    "combine reversed weights": (
        "acc = fmaf(topk_weights[(int64_t)t * k + j], widen_bf16(expert_out[row * H + h]), acc);\n      }\n      out[",
        "acc = fmaf(topk_weights[(int64_t)t * k + (k - 1 - j)], widen_bf16(expert_out[row * H + h]), acc);\n      }\n      out["),
    "combine drops last slot": (
        "      float acc = 0.0f;\n      for (int32_t j = 0; j < k; ++j) {",
        "      float acc = 0.0f;\n      for (int32_t j = 0; j < k - 1; ++j) {"),
    "combine truncates": (
        "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;",
        "if (lower > 0xFFFFu) upper += 1u;"),
    "combine ties round down": (
        "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;",
        "if (lower > 0x8000u) upper += 1u;"),
    "combine ties away from zero": (
        "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;",
        "if (lower >= 0x8000u) upper += 1u;"),
    "combine squares weight": (
        "acc = fmaf(topk_weights[(int64_t)t * k + j], widen_bf16(expert_out[row * H + h]), acc);\n      }\n      out[",
        "acc = fmaf(topk_weights[(int64_t)t * k + j] * topk_weights[(int64_t)t * k + j], widen_bf16(expert_out[row * H + h]), acc);\n      }\n      out["),
    "combine rounds the product first": (
        "acc = fmaf(topk_weights[(int64_t)t * k + j], widen_bf16(expert_out[row * H + h]), acc);\n      }\n      out[",
        "acc = acc + topk_weights[(int64_t)t * k + j] * widen_bf16(expert_out[row * H + h]);\n      }\n      out["),
    "partial ignores the rank": (
        "if (!id_is_expert(e, E) || e / m != r) continue; /* not an expert of rank r */",
        "if (!id_is_expert(e, E)) continue; /* not an expert of rank r */"),
    "partial rounds the product first": (
        "acc = fmaf(topk_weights[(int64_t)t * k + j], widen_bf16(expert_out[row * H + h]), acc);\n        }\n        partial",
        "acc = acc + topk_weights[(int64_t)t * k + j] * widen_bf16(expert_out[row * H + h]);\n        }\n        partial"),
    "partial walks slots backwards": (
        "for (int32_t j = 0; j < k; ++j) {\n          const int32_t e = topk_ids[(int64_t)t * k + j];\n          if (!id_is_expert(e, E) || e / m != r) continue; /* not",
        "for (int32_t j = k - 1; j >= 0; --j) {\n          const int32_t e = topk_ids[(int64_t)t * k + j];\n          if (!id_is_expert(e, E) || e / m != r) continue; /* not"),
    "partial segment starts one late": (
        "int64_t lo = rank_offsets[r], hi = rank_offsets[r + 1];",
        "int64_t lo = rank_offsets[r] + 1, hi = rank_offsets[r + 1];"),
    "partial ignores the expert cap": (
        "          if (row >= cap_expert) {\n            err |= ORACLE_ERR_EXPERT_CAP;\n            continue;\n          }\n          acc = fmaf(",
        "          if (row >= cap_expert + 1000000) {\n            err |= ORACLE_ERR_EXPERT_CAP;\n            continue;\n          }\n          acc = fmaf("),
    "home sum walks ranks backwards": (
        "for (int32_t r = 0; r < R; ++r) {\n        const int64_t s = token_rank_slot",
        "for (int32_t r = R - 1; r >= 0; --r) {\n        const int64_t s = token_rank_slot"),
    "home sum drops the last rank": (
        "for (int32_t r = 0; r < R; ++r) {\n        const int64_t s = token_rank_slot",
        "for (int32_t r = 0; r < R - 1; ++r) {\n        const int64_t s = token_rank_slot"),
    "home sum ignores the rank cap": (
        "        if (s >= cap_rank) {\n          err |= ORACLE_ERR_RANK_CAP;",
        "        if (s >= cap_rank + 1000000) {\n          err |= ORACLE_ERR_RANK_CAP;"),
    "padding rounds down": (
        "const int32_t run = (expert_counts[e] + align - 1) / align * align;",
        "const int32_t run = expert_counts[e] / align * align;"),
    "padding one row short": (
        "const int32_t run = (expert_counts[e] + align - 1) / align * align;",
        "const int32_t run = (expert_counts[e] + align - 2) / align * align;"),
    "masked blocks packed contiguously": (
        "expert_offsets[e + 1] = (e + 1) * block;",
        "expert_offsets[e + 1] = expert_offsets[e] + expert_counts[e];"),
    "masked block overflow kept": (
        "if (block > 0 && row >= (e + 1) * block) {",
        "if (block > 0 && row > (e + 1) * block) {"),
    "padding rows not marked": (
        "      expert_src_pair[row] = -1;\n  }\n  return err;",
        "      (void)0;\n  }\n  return err;"),
    "padding marks one row too many": (
        "row < end && row < cap_expert; ++row)",
        "row <= end && row < cap_expert; ++row)"),
    "mx exponent off by one (emax 7)": (
        "e = ex - 1 - 8;",
        "e = ex - 1 - 7;"),
    "mx ceiling of log2": (
        "e = ex - 1 - 8;",
        "e = ex - 8;"),
    "mx scale not clamped below": (
        "e = ex - 1 - 8;\n        if (e < -127) e = -127;",
        "e = ex - 1 - 8;\n        if (e < -160) e = -160;"),
    "mx4 scale not clamped below": (
        "e = ex - 1 - 2;\n        if (e < -127) e = -127;",
        "e = ex - 1 - 2;\n        if (e < -160) e = -160;"),
    "mx ties away from zero": (
        "e4m3_magnitude(c));\n          if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {",
        "e4m3_magnitude(c));\n          if (d <= best_d) {"),
    "mx4 ties away from zero": (
        "e2m1_magnitude(c));\n            if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {",
        "e2m1_magnitude(c));\n            if (d <= best_d) {"),
    "mx4 exponent off by one (emax 3)": (
        "e = ex - 1 - 2;",
        "e = ex - 1 - 3;"),
    "mx4 high nibble first": (
        "        if (i % 2 == 0)\n          out[i / 2] = (uint8_t)code;\n        else\n          out[i / 2] = (uint8_t)(out[i / 2] | (code << 4));",
        "        if (i % 2 == 0)\n          out[i / 2] = (uint8_t)(code << 4);\n        else\n          out[i / 2] = (uint8_t)(out[i / 2] | code);"),
    "e2m1 subnormal halved": (
        "if (ef == 0) return 0.5 * mf;",
        "if (ef == 0) return 0.25 * mf;"),
    "mx4 drops the sign": (
        "        code |= (v[i] >> 15) << 3;",
        "        code |= 0;"),
    "mx drops the sign": (
        "out[i] = (uint8_t)(((v[i] >> 15) << 7) | best);",
        "out[i] = (uint8_t)best;"),
    "mx ignores NaN blocks": (
        "if (!isfinite(a)) special = 1;\n        else if (a > amax) amax = a;\n      }\n      if (special) {",
        "if (!isfinite(a)) special = 0;\n        else if (a > amax) amax = a;\n      }\n      if (special) {"),
    "mx4 ignores NaN blocks": (
        "if (!isfinite(a)) special = 1;\n        else if (a > amax) amax = a;\n      }\n      int e = -127;",
        "if (!isfinite(a)) special = 0;\n        else if (a > amax) amax = a;\n      }\n      int e = -127;"),
    "e4m3 subnormals one binade low": (
        "if (ef == 0) return ldexp((double)mf, -9);",
        "if (ef == 0) return ldexp((double)mf, -10);"),
    "nv4 scale from amax / 4": (
        "nearest_code(amax / 6.0, 0x7E, e4m3_magnitude)",
        "nearest_code(amax / 4.0, 0x7E, e4m3_magnitude)"),
    "nv4 scale may reach the NaN code": (
        "nearest_code(amax / 6.0, 0x7E, e4m3_magnitude)",
        "nearest_code(amax / 6.0, 0x7F, e4m3_magnitude)"),
    "nearest code ties to odd": (
        "if (dc < db || (dc == db && c % 2 == 0)) best = c;",
        "if (dc < db || (dc == db && c % 2 == 1)) best = c;"),
    "nv4 zero scale not special": (
        "else if (s > 0.0)\n          code = nearest_code",
        "else\n          code = nearest_code"),
    "nv4 high nibble first": (
        "if ((i & 1) == 0)\n          out[i >> 1] = (uint8_t)code;\n        else\n          out[i >> 1] |= (uint8_t)(code << 4);",
        "if ((i & 1) == 0)\n          out[i >> 1] = (uint8_t)(code << 4);\n        else\n          out[i >> 1] |= (uint8_t)code;"),
    "nv4 drops the sign": (
        "code |= (int)(v[i] >> 15) << 3; /* the sign */",
        "code |= 0;"),
    "nv4 ignores NaN blocks": (
        "if (!isfinite(a)) nonfinite = 1;",
        "if (!isfinite(a)) nonfinite = 0;"),
    "f64 combine rounds products to float": (
        "acc += (double)topk_weights[(int64_t)t * k + j] * (double)widen_bf16(expert_out[row * H + h]);",
        "acc += (double)(topk_weights[(int64_t)t * k + j] * widen_bf16(expert_out[row * H + h]));"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    find, repl = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation site for {name!r} not found exactly once"
    mutated = tmp_path / "moe_oracle.c"
    mutated.write_text(src.replace(find, repl))
    hdr = os.path.join(os.path.dirname(SRC), "moe_oracle.h")
    (tmp_path / "moe_oracle.h").write_text(open(hdr).read())
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    str(mutated), "-o", str(lib), "-lm"], check=True)
    # Run the pins in a child process: a broken oracle may write out of bounds.
    script = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import oracle, pins\n"
        "failed = []\n"
        "with oracle.use_library(%r):\n"
        "    for pin in pins.PINS:\n"
        "        try:\n"
        "            pin()\n"
        "        except (AssertionError, IndexError, ValueError):\n"
        "            failed.append(pin.__name__)\n"
        "print('FAILED_PINS', ' '.join(failed))\n"
    ) % (ROOT, TESTS, str(lib))
    proc = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True,
                          timeout=300)
    if proc.returncode != 0:
        return  # the broken oracle crashed the pin run: caught
    line = [x for x in proc.stdout.splitlines() if x.startswith("FAILED_PINS")][-1]
    assert line.split()[1:], f"no pin caught the mutant {name!r}"
