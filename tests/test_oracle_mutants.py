"""Planted mistakes in the oracle (on the CPU) must each fail a pin.

Each mutant is a copy of oracle/moe_ep_oracle.c with one plausible mistake
(a wrong order, a dropped term, a wrong index, a fused multiply-add, the
wrong tie rule ...), compiled with gcc into a temporary directory. The pins
of test_oracle_pins.py are run against it; at least one must fail. This
shows the pins are tight enough to catch what a plausible bug would change.
"""
import multiprocessing as mp
import subprocess
import time

import pytest

import oracle
from oracle import build as obuild
import test_oracle_fp4 as fp4pins
import test_oracle_fp8 as fp8pins
import test_oracle_pins as pins
import test_oracle_sanitize as sanpins

MUTANTS = {
    "slots_descending_tokens": (
        "        for (int64_t t = 0; t < T; ++t) {\n            /* entries of token t",
        "        for (int64_t t = T - 1; t >= 0; --t) {\n            /* entries of token t"),
    "picks_reverse_router_order": (
        "            int32_t j = 0;\n            for (int32_t k = 0; k < K; ++k) {",
        "            int32_t j = 0;\n            for (int32_t k = K - 1; k >= 0; --k) {"),
    "padding_not_filtered": (
        "                if (id < 0 || id >= E)\n                    continue;\n                if (id / e_local == d)",
        "                if (id >= E)\n                    continue;\n                if (id / e_local == d)"),
    "global_instead_of_local_id": (
        "send_eloc[meta + j] = id - d * e_local;",
        "send_eloc[meta + j] = id;"),
    "weight_of_wrong_pick": (
        "send_w[meta + j] = topk_weights[t * K + k];",
        "send_w[meta + j] = topk_weights[t * K + (k + 1) % K];"),
    "batch_sources_descending": (
        "    for (int32_t s = 0; s < W; ++s) {\n        int64_t cnt = recv_cnt[s * cnt_rank_stride];\n        if (cnt < 0 || cnt > cap) {\n            err |= ORACLE_ERR_CNT;\n            cnt = cnt < 0 ? 0 : cap;\n        }\n        for (int64_t slot = 0; slot < cnt; ++slot) {\n            for (int32_t j = 0; j < slots; ++j) {\n                int32_t e = recv_eloc",
        "    for (int32_t s = W - 1; s >= 0; --s) {\n        int64_t cnt = recv_cnt[s * cnt_rank_stride];\n        if (cnt < 0 || cnt > cap) {\n            err |= ORACLE_ERR_CNT;\n            cnt = cnt < 0 ? 0 : cap;\n        }\n        for (int64_t slot = 0; slot < cnt; ++slot) {\n            for (int32_t j = 0; j < slots; ++j) {\n                int32_t e = recv_eloc"),
    "reduce_fused_multiply_add": (
        "                    float prod = y * wgt;\n                    acc = acc + prod;",
        "                    acc = __builtin_fmaf(y, wgt, acc);"),
    "reduce_drops_last_pick": (
        "                for (int32_t j = 0; j < slots; ++j) {\n                    int64_t at",
        "                for (int32_t j = 0; j < slots - 1; ++j) {\n                    int64_t at"),
    "reduce_weight_ignored": (
        "                    float prod = y * wgt;",
        "                    float prod = y;"),
    "round_half_up": (
        "(dropped == 0x8000u && (kept & 1u))",
        "(dropped == 0x8000u)"),
    "truncate_instead_of_round": (
        "        kept += 1u;                /* may carry",
        "        kept += 0u;                /* may carry"),
    "unpack_skips_first_rank": (
        "            for (int32_t d = 0; d < W; ++d) {\n                int32_t slot = token_slot[t * W + d];",
        "            for (int32_t d = 1; d < W; ++d) {\n                int32_t slot = token_slot[t * W + d];"),
    "reduce_row_of_first_pick": (
        "                    int32_t row = recv_row[at];",
        "                    int32_t row = recv_row[at - j];"),
    "quant_scale_wrong_divisor": (
        "const float s = amax > 0.0f ? amax / 448.0f : 1.0f;",
        "const float s = amax > 0.0f ? amax / 447.0f : 1.0f;"),
    "quant_multiplies_by_scale": (
        "const float y = v / s;",
        "const float y = v * s;"),
    "quant_times_448_over_amax": (
        "const float y = v / s;",
        "const float y = v * (amax > 0.0f ? 448.0f / amax : 1.0f);"),
    "quant_times_reciprocal_of_scale": (
        "const float y = v / s;",
        "const float y = v * (1.0f / s);"),
    "quant_sign_from_product": (
        "(uint8_t)((c & 0x7Fu) | (signbit(v) ? 0x80u : 0u));",
        "c;"),
    "fp4_amax_takes_nan": (
        "float v = fabsf(oracle_bf16_to_f32(x[t * x_row_stride + h]));\n                if (v > amax)\n                    amax = v;\n            }\n            const uint8_t s8",
        "float v = fabsf(oracle_bf16_to_f32(x[t * x_row_stride + h]));\n                if (!(v <= amax))\n                    amax = v;\n            }\n            const uint8_t s8"),
    "e4m3_subnormal_round_half_up": (
        "const double m = rint(a * 512.0);",
        "const double m = floor(a * 512.0 + 0.5);"),
    "e4m3_normal_round_half_up": (
        "double m = rint(ldexp(a, 3 - e));",
        "double m = floor(ldexp(a, 3 - e) + 0.5);"),
    "e4m3_wrong_bias": (
        "return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | ((int)m - 8)));",
        "return (uint8_t)(sign | (uint8_t)(((e + 8) << 3) | ((int)m - 8)));"),
    "quant_amax_without_abs": (
        "(g + 1) * group && h < H; ++h) {\n                float v = fabsf(oracle_bf16_to_f32(x[t * x_row_stride + h]));",
        "(g + 1) * group && h < H; ++h) {\n                float v = oracle_bf16_to_f32(x[t * x_row_stride + h]);"),
    "fp4_amax_without_abs": (
        "h < b * 16 + 16; ++h) {\n                float v = fabsf(oracle_bf16_to_f32(x[t * x_row_stride + h]));",
        "h < b * 16 + 16; ++h) {\n                float v = oracle_bf16_to_f32(x[t * x_row_stride + h]);"),
    "expert_rows_transposed_stride": (
        "e * y_expert_stride + row * y_row_stride + h",
        "row * y_expert_stride + e * y_row_stride + h"),
    "sanitize_keeps_negative_ids": (
        "if (e >= 0 && e < e_local)\n                        v = e;",
        "if (e < e_local)\n                        v = e;"),
    "e4m3_saturates_to_nan": (
        "    if (a >= 448.0)\n        return (uint8_t)(sign | 0x7Eu);",
        "    if (a >= 448.0)\n        return (uint8_t)(sign | 0x7Fu);"),
    "e2m1_nan_saturates": (
        "    if (f != f)\n        return sign;",
        "    if (f != f)\n        return (uint8_t)(sign | 7);"),
    "capacities_slots_is_k": (
        "    *slots = K < e_local ? K : e_local;",
        "    *slots = K;"),
    "capacities_expert_cap_is_cap": (
        "    *expert_cap = max_num_tokens * (int64_t)W;",
        "    *expert_cap = max_num_tokens;"),
    "reduce_rounds_every_add_to_bf16": (
        "                    acc = acc + prod;",
        "                    acc = oracle_bf16_to_f32(oracle_f32_to_bf16(acc + prod));"),
    "unpack_rounds_every_add_to_bf16": (
        "                acc = acc + load_elem(back, dtype,\n                                      d * back_rank_stride + slot * back_row_stride + h);",
        "                acc = oracle_bf16_to_f32(oracle_f32_to_bf16(acc + load_elem(back, dtype,\n                                      d * back_rank_stride + slot * back_row_stride + h)));"),
    "sanitize_keeps_out_of_range_ids": (
        "if (e >= 0 && e < e_local)\n                        v = e;\n                }\n                out[",
        "if (e >= 0)\n                        v = e;\n                }\n                out["),
    "sanitize_out_of_range_not_flagged": (
        "                    if (e >= e_local)\n                        err |= ORACLE_ERR_ELOC;\n                    if (e >= 0 && e < e_local)\n                        v = e;",
        "                    if (e >= 0 && e < e_local)\n                        v = e;"),
    "sanitize_keeps_row_past_count": (
        "                if (slot < cnt) {\n                    int32_t e = recv_eloc",
        "                if (slot <= cnt) {\n                    int32_t e = recv_eloc"),
    "e2m1_ties_to_odd": (
        "(dc == db && (c & 1) == 0)",
        "(dc == db && (c & 1) == 1)"),
    "e2m1_saturates_to_4": (
        "        return (uint8_t)(sign | 7);  /* would tie",
        "        return (uint8_t)(sign | 6);  /* would tie"),
    "fp4_nibbles_swapped": (
        "(uint8_t)(c0 | (c1 << 4))",
        "(uint8_t)(c1 | (c0 << 4))"),
    "fp4_scale_divisor": (
        "oracle_f32_to_e4m3(amax / 6.0f)",
        "oracle_f32_to_e4m3(amax / 4.0f)"),
    "fp4_codes_from_unrounded_scale": (
        "            const float s = oracle_e4m3_to_f32(s8);",
        "            const float s = amax / 6.0f;"),
    "fp4_times_reciprocal_of_scale": (
        "const float y0 = s > 0.0f ? v0 / s : 0.0f;\n                const float y1 = s > 0.0f ? v1 / s : 0.0f;",
        "const float y0 = s > 0.0f ? v0 * (1.0f / s) : 0.0f;\n                const float y1 = s > 0.0f ? v1 * (1.0f / s) : 0.0f;"),
    "pick_ranks_one_based": (
        "                send_rank[at] = send_ecnt[(int64_t)d * e_local + e];\n                send_ecnt[(int64_t)d * e_local + e] += 1;",
        "                send_ecnt[(int64_t)d * e_local + e] += 1;\n                send_rank[at] = send_ecnt[(int64_t)d * e_local + e];"),
    "fp8_zero_group_scale_zero": (
        "            const float s = amax > 0.0f ? amax / 448.0f : 1.0f;",
        "            const float s = amax > 0.0f ? amax / 448.0f : 0.0f;"),
    "fp8_amax_takes_nan": (
        "                if (v > amax)\n                    amax = v;\n            }\n            const float s = amax",
        "                if (!(v <= amax))\n                    amax = v;\n            }\n            const float s = amax"),
    "reduce_sum_starts_at_negative_zero": (
        "                float acc = 0.0f;\n                for (int32_t j = 0; j < slots; ++j) {",
        "                float acc = -0.0f;\n                for (int32_t j = 0; j < slots; ++j) {"),
    "unpack_sum_starts_at_negative_zero": (
        "            float acc = 0.0f;\n            for (int32_t d = 0; d < W; ++d) {",
        "            float acc = -0.0f;\n            for (int32_t d = 0; d < W; ++d) {"),
    "pack_unused_weight_negative_zero": (
        "                send_w[meta + j] = 0.0f;",
        "                send_w[meta + j] = -0.0f;"),
    "pack_no_pair_slot_zero": (
        "                token_slot[t * W + d] = -1;\n                continue;",
        "                token_slot[t * W + d] = 0;\n                continue;"),
    "pack_slots_count_picks": (
        "            count += 1;",
        "            count += npicks;"),
    "expert_num_tokens_unclamped": (
        "        expert_num_tokens[e] = (int32_t)(n[e] < expert_cap ? n[e] : expert_cap);",
        "        expert_num_tokens[e] = (int32_t)n[e];"),
    "batch_padding_pick_flagged": (
        "                if (e < 0) {\n                    recv_row[at] = -1;\n                    continue;",
        "                if (e < 0) {\n                    err |= ORACLE_ERR_ELOC;\n                    recv_row[at] = -1;\n                    continue;"),
    "pick_ranks_shared_across_destinations": (
        "                send_rank[at] = send_ecnt[(int64_t)d * e_local + e];\n                send_ecnt[(int64_t)d * e_local + e] += 1;",
        "                send_rank[at] = send_ecnt[e];\n                send_ecnt[e] += 1;"),
    "pick_ranks_columns_reversed": (
        "            for (int32_t j = 0; j < slots; ++j) {\n                int64_t at = ((int64_t)d * cap + slot) * slots + j;\n                int32_t e = send_eloc[at];",
        "            for (int32_t j = slots - 1; j >= 0; --j) {\n                int64_t at = ((int64_t)d * cap + slot) * slots + j;\n                int32_t e = send_eloc[at];"),
    "bf16_nan_drops_quiet_bit": (
        "return (uint16_t)(kept | 0x0040u);",
        "return (uint16_t)kept;"),
    "bf16_nan_rounded_like_numbers": (
        "    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)\n        return (uint16_t)(kept | 0x0040u);\n",
        ""),
    "bf16_nan_canonical": (
        "return (uint16_t)(kept | 0x0040u);",
        "return (uint16_t)0x7FC0u;"),
    "e4m3_decode_wrong_bias": (
        "v = ldexp(8.0 + f, e - 10);",
        "v = ldexp(8.0 + f, e - 9);"),
}


def _pin_battery():
    """Fast subset of the pins, each a zero-argument callable."""
    return [
        pins.test_golden_pack,
        pins.test_golden_batch,
        lambda: pins.test_golden_reduce("bf16"),
        lambda: pins.test_golden_reduce("f32"),
        lambda: pins.test_golden_unpack("bf16"),
        pins.test_golden_bf16_rounding,
        pins.test_golden_bf16_nan,
        lambda: pins.test_golden_products_rounded_before_add("bf16"),
        lambda: pins.test_pack_exhaustive_micro(2, 2),
        pins.test_combine_dense_brute_force_tiny,
        lambda: pins.test_identity_round_trip_returns_a1(1),
        lambda: pins.test_power_of_two_experts(1),
        lambda: pins.test_invariants_full_size_metadata(1),
        fp8pins.test_every_finite_code_round_trips,
        fp8pins.test_midpoints_round_to_even_and_neighbours_to_nearest,
        fp8pins.test_golden_quantized_row,
        fp8pins.test_quantize_dequantize_error_bound,
        sanpins.test_sanitize_hand_example,
        fp4pins.test_e4m3_decoder_matches_definition_and_torch,
        fp4pins.test_e2m1_every_code_round_trips,
        fp4pins.test_e2m1_midpoints_neighbours_and_random_match_exact_rounding,
        fp4pins.test_golden_fp4_rows,
        fp4pins.test_fp4_dequantisation_error_bound,
        fp4pins.test_fp4_nonfinite_inputs,
        fp8pins.test_fp8_nonfinite_inputs,
        lambda: sanpins.test_sanitize_matches_brute_force_from_routing(4, 8, 3),
        pins.test_error_bits,
        lambda: pins.test_reduce_sums_start_at_positive_zero("f32"),
        pins.test_golden_pick_ranks,
        pins.test_pick_ranks_random_micro,
        lambda: pins.test_pick_ranks_give_the_receive_rows(2),
    ]


def _child(libs, conn):
    """Runs the pin battery against each (name, library) in turn and reports
    ("start", name) before and ("done", name, failing pins) after each. The
    reports go through a pipe, written at once, so none is lost when a
    mutant crashes the process."""
    import faulthandler
    faulthandler.disable()          # a crashing mutant is an expected outcome
    for name, lib_path in libs:
        conn.send(("start", name))
        failed = 0
        with oracle.use_library(lib_path):
            for fn in _pin_battery():
                try:
                    fn()
                except Exception:   # an assertion or a rejected call
                    failed += 1
                    break           # one failing pin is enough
        conn.send(("done", name, failed))
    conn.close()


def _failing_pins(libs, limit_s=600):
    """{name: failing pins} for each (name, library), all in one spawned,
    CPU-only process, which saves starting one per mutant. A library that
    crashes the process counts as caught (1000 failing pins), and the ones
    after it run in a new process. Spawned, not forked: the parent may
    already run torch's CPU thread pool, which a forked child cannot use."""
    ctx = mp.get_context("spawn")
    results = {}
    pending = list(libs)
    t0 = time.monotonic()
    while pending:
        rd, wr = ctx.Pipe(duplex=False)
        p = ctx.Process(target=_child, args=(pending, wr))
        p.start()
        wr.close()                  # the child holds the only write end
        current = None
        while True:
            if time.monotonic() - t0 > limit_s:
                p.kill()
                p.join()
                raise AssertionError(f"pin batteries did not finish (at {current})")
            if not rd.poll(1):
                if p.is_alive():
                    continue
                if not rd.poll(0):
                    break
            try:
                msg = rd.recv()
            except EOFError:        # the child has ended and all is read
                break
            if msg[0] == "start":
                current = msg[1]
            else:
                results[msg[1]] = msg[2]
                current = None
        p.join()
        rd.close()
        if current is not None:     # the process died inside this battery
            results[current] = 1_000
        left = [(n, lib) for n, lib in pending if n not in results]
        if len(left) == len(pending):
            raise AssertionError(f"the pin battery process ended without running "
                                 f"(exit code {p.exitcode})")
        pending = left
    return results


def _compile(name, src, tmp_dir):
    c = tmp_dir / f"{name}.c"
    c.write_text(src)
    so = tmp_dir / f"{name}.so"
    subprocess.run(["gcc", *obuild.CFLAGS, "-o", str(so), str(c), "-lm"], check=True)
    return str(so)


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    src = open(obuild.SRC).read()
    tmp_dir = tmp_path_factory.mktemp("mutants")
    libs, procs = [], []
    for name in sorted(MUTANTS):    # the compilers run side by side
        old, new = MUTANTS[name]
        if src.count(old) != 1:
            continue                # reported by the test of that mutant
        c = tmp_dir / f"{name}.c"
        c.write_text(src.replace(old, new))
        so = tmp_dir / f"{name}.so"
        procs.append(subprocess.Popen(["gcc", *obuild.CFLAGS, "-o", str(so), str(c), "-lm"]))
        libs.append((name, str(so)))
    for pr in procs:
        assert pr.wait() == 0, "a mutant did not compile"
    return _failing_pins(libs)


def test_unmutated_copy_passes_battery(tmp_path):
    so = _compile("unmutated", open(obuild.SRC).read(), tmp_path)
    assert _failing_pins([("unmutated", so)]) == {"unmutated": 0}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_results):
    old, _ = MUTANTS[name]
    assert open(obuild.SRC).read().count(old) == 1, f"mutation site of {name} not unique"
    assert mutant_results[name] > 0, f"no pin caught mutant {name}"
