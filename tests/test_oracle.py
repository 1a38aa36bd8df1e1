"""The fp64 oracle against its pins (CPU only), and a check that the pins
would catch plausible mistakes planted in a copy of the oracle's source."""
import os
import shutil
import tempfile

import pytest

import oracle
import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle._load())


# Each planted mistake is a textual edit of pa_oracle.c of the kind a careless
# transcription of the definition would make.
MUTATIONS = [
    ("causal bound off by one", "int32_t nk = (int32_t)p + 1;", "int32_t nk = (int32_t)p;"),
    ("top-left instead of bottom-right", "return (int64_t)ctx + (t - a->cu[r]);", "return (int64_t)(t - a->cu[r]) + (ctx > 0);"),
    ("wrong KV head of a query head", "int32_t g = h / G;", "int32_t g = h % a->hkv;"),
    ("dropped scale", "scores[i - k0] = a->scale * dot;", "scores[i - k0] = dot;"),
    ("max subtracted with the wrong sign", "scores[i] = exp(scores[i] - m);", "scores[i] = exp(m - scores[i]);"),
    ("missing normalisation", "for (int32_t d = 0; d < a->d; ++d) out_row[d] /= z;", ""),
    ("page offset from the wrong index", "int32_t off = i % a->bs;", "int32_t off = (i + 1) % a->bs;"),
    ("logical block from the wrong index", "int32_t lb = i / a->bs;", "int32_t lb = (i / a->bs + 1) % a->max_blocks;"),
    ("split weights with flipped exponent", "double w = l[n * max_parts + k] * exp2(m[n * max_parts + k] - M);",
     "double w = l[n * max_parts + k] * exp2(M - m[n * max_parts + k]);"),
    ("partition bound off by one", "int32_t parts = p < 0 ? 0 : (int32_t)((p + partition_size) / partition_size);",
     "int32_t parts = p < 0 ? 0 : (int32_t)((p + partition_size - 1) / partition_size);"),
    ("partial statistic not in log2 space", "scores[i] *= LOG2E; /* log2-space score */", ""),
    ("cache write: K and V swapped", "memcpy((char *)key_cache + dst, (const char *)key", "memcpy((char *)key_cache + dst, (const char *)value"),
    ("cache write: block offset dropped", "size_t dst = ((size_t)blk * block_size + (size_t)off) * row;", "size_t dst = ((size_t)blk * block_size) * row;"),
    ("block-table view: wrong page order", "v * ratio + j", "v + j * ratio"),
    ("V read through the K cache", "out_row[d] += scores[i] * load_kv(a, a->vc,", "out_row[d] += scores[i] * load_kv(a, a->kc,"),
    ("block copy: source and destination ids swapped",
     "int64_t s = pairs[2 * i], d = pairs[2 * i + 1];", "int64_t d = pairs[2 * i], s = pairs[2 * i + 1];"),
    ("block copy: V taken from the K pool", "memcpy((char *)dst_value + d * block_bytes, (const char *)src_value",
     "memcpy((char *)dst_value + d * block_bytes, (const char *)src_key"),
    ("sink left out of the denominator", "double z = a->sinks ? exp(sink - m) : 0.0;", "double z = 0.0;"),
    ("sink merged in natural units", "double sink2 = sinks ? (double)sinks[h] * LOG2E : -INFINITY;",
     "double sink2 = sinks ? (double)sinks[h] : -INFINITY;"),
    ("e4m3: exponent bias 8", "mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("e4m3: subnormal exponent", "mag = ldexp((double)m / 8.0, -6);", "mag = ldexp((double)m / 8.0, -7);"),
    ("e4m3: ties away from zero", "(err == best_err && (c & 1) == 0)", "(err == best_err)"),
    ("e4m3: overflow to NaN", "if (a > 448.0) a = 448.0; /* saturate (infinities too) */",
     "if (a > 448.0) return (uint8_t)(sign | 0x7F);"),
    ("e4m3: sign dropped", "return (uint8_t)(sign | best);", "return (uint8_t)best;"),
    ("fp8 write: scale multiplies", "quotient_f32(load_elem(key, src, dtype), (double)k_scale[g])",
     "quotient_f32(load_elem(key, src, dtype), 1.0 / (double)k_scale[g])"),
    ("fp8 write: V with the K scale", "quotient_f32(load_elem(value, src, dtype), (double)v_scale[g])",
     "quotient_f32(load_elem(value, src, dtype), (double)k_scale[g])"),
    ("fp8 write: quotient not rounded to float32", "static float quotient_f32(double x, double s) { return (float)(x / s); }",
     "static double quotient_f32(double x, double s) { return x / s; }"),
    ("fp8 read: V with the K scale", "load_kv(a, a->vc, a->v_scale,", "load_kv(a, a->vc, a->k_scale,"),
    ("fp8 read: scale of the wrong head", "* (double)scale[g];", "* (double)scale[0];"),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistakes(name, old, new, tmp_path):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mutant = tmp_path / "pa_oracle.c"
    mutant.write_text(src.replace(old, new))
    shutil.copy(os.path.join(os.path.dirname(oracle._SRC), "pa_oracle.h"), tmp_path / "pa_oracle.h")
    so = oracle.build(force=True, out_path=str(tmp_path / "libmutant.so"), src_path=str(mutant))
    lib = oracle._load(so)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"
