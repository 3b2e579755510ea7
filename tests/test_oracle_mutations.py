"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one (no GPU).  Each mutant is a textual edit of oracle.c built
into a temporary library; the original is never modified."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

# the store of one quantized (token, head) row, as each quantizing append writes it
_QROW = ("int64_t block = slots[t] {div} block_size, off = slots[t] {mod} block_size;\n"
         "    for (int32_t h = 0; h < num_kv_heads; ++h) {{\n"
         "      size_t src = ((size_t)t * num_kv_heads + h) * head_dim;\n"
         "      size_t srow = ((size_t)block * num_kv_heads + h) * block_size + off;\n"
         "      oracle_quantize_row_{kind}(")

MUTANTS = {
    "scale dropped from the scores": ("z[i] = scale * dot;", "z[i] = dot;"),
    "GQA head mapped round-robin": (
        "int32_t kvh = h / group;\n    size_t n =", "int32_t kvh = h % num_kv_heads;\n    size_t n ="),
    "prefill GQA head mapped round-robin": (
        "int32_t kvh = h / group;\n    double* K", "int32_t kvh = h % num_kv_heads;\n    double* K"),
    "offset in block taken from the block index": (
        "block_size + i % block_size;\n    double sk", "block_size + i / block_size;\n    double sk"),
    "softmax not normalised": ("double w = z[i] / total;", "double w = z[i];"),
    "binary16 exponent bias off by one": ("expo - 25);", "expo - 24);"),
    "binary16 subnormal scale wrong": ("ldexp((double)frac, -24);", "ldexp((double)frac, -23);"),
    "bfloat16 shifted wrong": ("(uint32_t)b << 16;", "(uint32_t)b << 15;"),
    "int8 key scale dropped": ("row * head_dim + d) * sk;", "row * head_dim + d);"),
    "newest token excluded from attention": (
        "oracle_attention_dense(qv, K, V, ctx,", "oracle_attention_dense(qv, K, V, ctx - 1,"),
    "decode slot offset from block index": (
        "slots[s] = (int64_t)block * block_size + pos % block_size;",
        "slots[s] = (int64_t)block * block_size + pos / block_size;"),
    "append block/offset swapped": (
        "int64_t block = slots[t] / block_size, off = slots[t] % block_size;\n    for (int32_t h = 0; h < num_kv_heads; ++h) {\n      size_t src = ((size_t)t * num_kv_heads + h) * row;",
        "int64_t block = slots[t] % block_size, off = slots[t] / block_size;\n    for (int32_t h = 0; h < num_kv_heads; ++h) {\n      size_t src = ((size_t)t * num_kv_heads + h) * row;"),
    "quantizer truncates": ("float c = rintf(r);", "float c = truncf(r);"),
    "quantizer range 128": ("volatile float ratio = a / 127.0f;", "volatile float ratio = a / 128.0f;"),
    "values mixed from keys": ("out[d] += w * V[i * head_dim + d];", "out[d] += w * K[i * head_dim + d];"),
    "running minimum instead of maximum": ("if (z[i] > m) m = z[i];", "if (z[i] < m) m = z[i];"),
    "gather offset from block index": (
        "block_size + i % block_size;\n        size_t dst_row", "block_size + i / block_size;\n        size_t dst_row"),
    "binary16 rounding truncates": ("double n = nearbyint(a / quantum);", "double n = floor(a / quantum);"),
    "prefill position counted from the chunk start": (
        "int32_t pos = context_lens[s] - t_s + (int32_t)(tok - query_start[s]);",
        "int32_t pos = (int32_t)(tok - query_start[s]);"),
    "prefill query excludes its own position": ("int32_t n = pos + 1;                    /*",
                                                "int32_t n = pos;                    /*"),
    "prefill token given to the previous sequence": (
        "while (query_start[s + 1] <= tok) ++s;", "while (query_start[s + 1] < tok) ++s;"),
    "fp8 exponent bias off by one": ("ldexp(8.0 + frac, expo - 10)", "ldexp(8.0 + frac, expo - 9)"),
    "fp8 subnormals scaled as normals": ("ldexp((double)frac, -9)", "ldexp((double)frac, -10)"),
    "fp8 ties to odd": ("(err == best_err && (c & 1) == 0)", "(err == best_err && (c & 1) == 1)"),
    "fp8 quantizer range 240": ("volatile float ratio = a / 448.0f;",
                                "volatile float ratio = a / 240.0f;"),
    "fp8 scales ignored by attention": ("if (dtype == OR_I8 || dtype == OR_FP8) {\n      sk",
                                        "if (dtype == OR_I8) {\n      sk"),
    "window one row too short": ("int32_t first = window > 0 && ctx > window ? ctx - window : 0;",
                                 "int32_t first = window > 0 && ctx > window ? ctx - window + 1 : 0;"),
    "window start not skipped inside its block": ("K + skip, V + skip, n,", "K, V, n,"),
    "int4 nibbles swapped": ("packed[e / 2] |= (uint8_t)(e % 2 ? nib << 4 : nib);",
                             "packed[e / 2] |= (uint8_t)(e % 2 ? nib : nib << 4);"),
    "int4 offset 7": ("uint8_t nib = (uint8_t)((int)c + 8);", "uint8_t nib = (uint8_t)((int)c + 7);"),
    "int4 range 8": ("volatile float ratio = a / 7.0f;", "volatile float ratio = a / 8.0f;"),
    "int4 one scale per row": ("size_t g = row * (head_dim / OR_I4_GROUP) + d / OR_I4_GROUP;",
                               "size_t g = row * (head_dim / OR_I4_GROUP);"),
    "int8 V pool quantized from the K row": ("oracle_quantize_row_int8(v_new + src",
                                             "oracle_quantize_row_int8(k_new + src"),
    "fp8 K pool quantized from the V row": ("oracle_quantize_row_fp8(k_new + src",
                                            "oracle_quantize_row_fp8(v_new + src"),
    "int4 K pool quantized from the V row": ("oracle_quantize_row_int4(k_new + src",
                                             "oracle_quantize_row_int4(v_new + src"),
    **{f"{kind} append block/offset swapped": (
        _QROW.format(div="/", mod="%", kind=kind), _QROW.format(div="%", mod="/", kind=kind))
       for kind in ("int8", "fp8", "int4")},
    **{f"{kind} append writes the pad slot's token to the next slot": (
        f"if (slots[t] < 0) continue;\n    int64_t block = slots[t] / block_size, off = slots[t] % block_size;\n    for (int32_t h = 0; h < num_kv_heads; ++h) {{\n      size_t src = ((size_t)t * num_kv_heads + h) * head_dim;\n      size_t srow = ((size_t)block * num_kv_heads + h) * block_size + off;\n      oracle_quantize_row_{kind}(",
        f"if (slots[t] < 0) continue;\n    int64_t block = slots[t] / block_size, off = slots[t] % block_size;\n    for (int32_t h = 0; h < num_kv_heads; ++h) {{\n      size_t src = ((size_t)(t > 0 && slots[t - 1] < 0 ? t - 1 : t) * num_kv_heads + h) * head_dim;\n      size_t srow = ((size_t)block * num_kv_heads + h) * block_size + off;\n      oracle_quantize_row_{kind}(")
       for kind in ("int8", "fp8", "int4")},
    "dot product over half the head": (
        "for (int32_t d = 0; d < head_dim; ++d) dot += q[d] * K[i * head_dim + d];",
        "for (int32_t d = 0; d < head_dim / 2; ++d) dot += q[d] * K[i * head_dim + d];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site not found exactly once: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(output=lib_path, source=str(path))
    lib = oracle.load(lib_path)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, oracle.OracleError, ValueError, IndexError) as e:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant '{name}'"
