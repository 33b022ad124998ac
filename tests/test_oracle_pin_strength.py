"""Each plausible mistake planted in a copy of the oracle's C source (on the CPU,
never in the product) must make at least one pin fail."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "pkv_oracle.c")

# (name, original text, mutated text) -- each must occur exactly once
MUTATIONS = [
    ("gather_offset_off_by_one", "int64_t off = t % B;", "int64_t off = (t + 1) % B;"),
    ("gather_block_index", "int64_t blk = table[t / B];", "int64_t blk = table[t / B + (t >= B)];"),
    ("gqa_strided_grouping",
     "const int32_t h = g * G + j;\n        const int64_t base = ((int64_t)s * Hq + h) * D;\n"
     "        for (int32_t d = 0; d < D; ++d) qd[d] = pkvo_load_elem(q, dtype, base + d);",
     "const int32_t h = j * Hkv + g;\n        const int64_t base = ((int64_t)s * Hq + h) * D;\n"
     "        for (int32_t d = 0; d < D; ++d) qd[d] = pkvo_load_elem(q, dtype, base + d);"),
    ("fp8_gqa_strided_grouping",
     "const int32_t h = g * G + j;\n        const int64_t base = ((int64_t)s * Hq + h) * D;\n"
     "        for (int32_t d = 0; d < D; ++d) qd[d] = pkvo_load_elem(q, q_dtype, base + d);",
     "const int32_t h = j * Hkv + g;\n        const int64_t base = ((int64_t)s * Hq + h) * D;\n"
     "        for (int32_t d = 0; d < D; ++d) qd[d] = pkvo_load_elem(q, q_dtype, base + d);"),
    ("scale_dropped", "z[t] = scale * acc;", "z[t] = acc;"),
    ("no_normalisation", "double p = z[t] / denom;", "double p = z[t];"),
    ("values_from_keys", "if (rc == PKVO_OK) rc = pkvo_gather(V, v_cache, dtype, table, L, NB, Hkv, D, B, g);\n      for (int32_t j = 0; j < G",
     "if (rc == PKVO_OK) rc = pkvo_gather(V, k_cache, dtype, table, L, NB, Hkv, D, B, g);\n      for (int32_t j = 0; j < G"),
    ("causal_off_by_one", "const int32_t visible = L - Qs + i + 1;", "const int32_t visible = L - Qs + i;"),
    ("causal_sees_future", "const int32_t visible = L - Qs + i + 1;", "const int32_t visible = L;"),
    ("f16_subnormal_exponent", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    ("f16_normal_bias", "v = ldexp((double)(m | 0x400), e - 25);", "v = ldexp((double)(m | 0x400), e - 24);"),
    ("bf16_shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("reshape_skips_slot_zero",
     "if (slot < 0) continue;\n    if (slot >= NB * B) return PKVO_ERANGE;\n    const int64_t blk",
     "if (slot <= 0) continue;\n    if (slot >= NB * B) return PKVO_ERANGE;\n    const int64_t blk"),
    ("fp8_reshape_skips_slot_zero",
     "if (slot < 0) continue;\n    if (slot >= NB * B) return PKVO_ERANGE;\n    for (int32_t h",
     "if (slot <= 0) continue;\n    if (slot >= NB * B) return PKVO_ERANGE;\n    for (int32_t h"),
    ("reshape_k_into_v", "memcpy((char*)v_cache + dst, (const char*)value", "memcpy((char*)v_cache + dst, (const char*)key"),
    ("copy_reads_destination", "memcpy(snap + (size_t)(2 * i) * blk_bytes, kc + (size_t)pairs[2 * i] * blk_bytes",
     "memcpy(snap + (size_t)(2 * i) * blk_bytes, kc + (size_t)pairs[2 * i + 1] * blk_bytes"),
    ("swap_reads_destination_index", "(const char*)src_pools[p] + (size_t)pairs[2 * i] * (size_t)block_bytes",
     "(const char*)src_pools[p] + (size_t)pairs[2 * i + 1] * (size_t)block_bytes"),
    ("e4m3_exponent_bias", "else v = ldexp((double)(8 + m), e - 10);", "else v = ldexp((double)(8 + m), e - 9);"),
    ("e4m3_subnormal_scale", "if (e == 0) v = ldexp((double)m, -9);", "if (e == 0) v = ldexp((double)m, -10);"),
    ("e4m3_ties_to_odd", "(d == best_d && (c & 1) == 0)", "(d == best_d && (c & 1) == 1)"),
    ("e4m3_ties_away", "(d == best_d && (c & 1) == 0)", "(d == best_d)"),
    ("e4m3_inf_to_nan", "if (isinf(x)) return (uint8_t)(sign | 0x7e);", "if (isinf(x)) return (uint8_t)(sign | 0x7f);"),
    ("fp8_quantize_multiplies", "const float kq = load_f32(key, in_dtype, src) / k_scale[h];",
     "const float kq = load_f32(key, in_dtype, src) * k_scale[h];"),
    ("fp8_v_uses_k_scale", "const float vq = load_f32(value, in_dtype, src) / v_scale[h];",
     "const float vq = load_f32(value, in_dtype, src) / k_scale[h];"),
    ("fp8_decode_drops_k_scale", "        K[i] *= (double)k_scale[g];\n", ""),
    ("fp8_decode_v_scale_of_k", "V[i] *= (double)v_scale[g];", "V[i] *= (double)k_scale[g];"),
    ("fp8_prefill_v_scale_of_k", "V[e] *= (double)v_scale[g];", "V[e] *= (double)k_scale[g];"),
    ("fp8_prefill_drops_k_scale", "          K[e] *= (double)k_scale[g];\n", ""),
]

# the pins, called directly (parametrised ones with representative arguments)
CASES = [
    (pins.test_f16_widening_matches_numpy_for_every_bit_pattern, {}),
    (pins.test_bf16_widening_matches_torch_for_every_bit_pattern, {}),
    (pins.test_gather_reproduces_kwkr_kvcache_manager_example,
     {"case": pins.golden("kwkr_kvcache_manager.json")["cases"][0]}),
    (pins.test_decode_contiguous_case_matches_torch_sdpa, {"dtype": "bf16", "Hq": 8, "Hkv": 2}),
    (pins.test_decode_matches_brute_force_loops, {"B": 4}),
    (pins.test_decode_single_token_returns_its_value_exactly, {}),
    (pins.test_decode_equal_keys_give_mean_of_values, {}),
    (pins.test_tiny_workload_matches_sdpa, {}),
    (pins.test_prefill_matches_causal_sdpa_on_whole_sequences, {"dtype": "f32"}),
    (pins.test_reshape_and_cache_matches_numpy_scatter, {"dtype": "f32"}),
    (pins.test_copy_blocks_matches_numpy_indexing, {}),
    (pins.test_swap_blocks_matches_numpy_indexing, {}),
    (pins.test_e4m3_decode_matches_torch_for_every_code, {}),
    (pins.test_e4m3_spec_constants, {}),
    (pins.test_e4m3_encode_matches_torch_inside_range, {}),
    (pins.test_e4m3_encode_clips_beyond_range_and_keeps_nan, {}),
    (pins.test_e4m3_round_trip_every_finite_code, {}),
    (pins.test_reshape_and_cache_fp8_matches_torch_quantization, {"in_dtype": "bf16"}),
    (pins.test_decode_fp8_matches_sdpa_on_dequantized_values, {"q_dtype": "bf16"}),
    (pins.test_decode_fp8_single_token_returns_code_times_scale, {}),
    (pins.test_prefill_fp8_matches_causal_sdpa_on_dequantized_values, {"q_dtype": "bf16"}),
]


@pytest.mark.parametrize("name,orig,mut", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, orig, mut, tmp_path):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation anchor not unique for {name}"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(orig, mut))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-ffp-contract=off", "-shared", "-o",
                    str(lib), str(path), "-lm"], check=True)
    caught = []
    with oracle.use_library(str(lib)):
        for fn, kw in CASES:
            try:
                fn(**kw)
            except (AssertionError, oracle.OracleError):
                caught.append(fn.__name__)
    assert caught, f"no pin caught mutation {name}"


def test_unmutated_oracle_passes_every_case():
    for fn, kw in CASES:
        fn(**kw)
