"""Plant one mistake at a time in a copy of the oracle's C source and check
that at least one pin fails for it: the pins are strong enough to catch a
dropped term, a wrong sign, a wrong index or a swapped operand.  CPU only;
every mutant stays within the arrays the original reads."""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from oracle_pins import ALL_PINS

MUTANTS = [
    ("scale 1/D instead of 1/sqrt(D)", "1.0 / sqrt((double)D)", "1.0 / (double)D"),
    ("exponent sign flipped", "exp(scores[j] - m)", "exp(m - scores[j])"),
    ("row max not subtracted", "exp(scores[j] - m)", "exp(scores[j])"),
    ("normalisation dropped", "scores[j] /= z;", "(void)z;"),
    ("causal window misses the diagonal", "causal ? (int64_t)i + 1", "causal ? (int64_t)i"),
    ("GQA head as h % H_kv (prefill)", "const int g = (int)(((int64_t)h * H_kv) / H_q); /* GQA kv head */\n\n        const uint16_t* qrow = q + (((int64_t)b",
     "const int g = (int)(h % H_kv); /* GQA kv head */\n\n        const uint16_t* qrow = q + (((int64_t)b"),
    ("GQA head as h % H_kv (decode)", "const int g = (int)(((int64_t)h * H_kv) / H_q); /* GQA kv head */\n          const uint16_t* qrow",
     "const int g = (int)(h % H_kv); /* GQA kv head */\n          const uint16_t* qrow"),
    ("value rows read from K", "vr[j] = v + off;", "vr[j] = k + off;"),
    ("decode slot offset shifted", "t % block_size) * D;", "(t + 1) % block_size) * D;"),
    ("decode value rows read from K cache", "vr[t] = v_cache + off;", "vr[t] = k_cache + off;"),
    ("binary16 exponent bias off by one", "e - 25", "e - 24"),
    ("binary16 subnormal scale", "ldexp((double)f, -24)", "ldexp((double)f, -23)"),
    ("LSE without the max", "*lse = m + log(z);", "*lse = log(z);"),
    ("score of key 0 skipped in max", "double m = scores[0];", "double m = scores[n - 1];\n  if (n > 1) m = scores[1];"),
    ("append: in-block offset shifted", "const int64_t off = slot % block_size;",
     "const int64_t off = (slot + 1) % block_size;"),
    ("append: slot 0 treated as padding", "if (slot < 0 || slot >= capacity) continue;",
     "if (slot <= 0 || slot >= capacity) continue;"),
    ("append: heads swapped", "uint16_t* kd = k_cache + ((block * H_kv + h) * block_size + off) * (int64_t)D;",
     "uint16_t* kd = k_cache + ((block * H_kv + (H_kv - 1 - h)) * block_size + off) * (int64_t)D;"),
    ("rope table: frequency exponent -i/D", "pow(theta, -2.0 * (double)i / (double)D)",
     "pow(theta, -1.0 * (double)i / (double)D)"),
    ("rope table: cos and sin swapped", "cos_out[(int64_t)p * half + i] = cos(angle);",
     "cos_out[(int64_t)p * half + i] = sin(angle);"),
    ("rope: first-half sign flipped", "o[i] = y[i] * c[i] - y[i + half] * s[i];",
     "o[i] = y[i] * c[i] + y[i + half] * s[i];"),
    ("rope: second-half sign flipped", "o[i + half] = y[i + half] * c[i] + y[i] * s[i];",
     "o[i + half] = y[i + half] * c[i] - y[i] * s[i];"),
    ("rope: adjacent pairs instead of split halves", "o[i] = y[i] * c[i] - y[i + half] * s[i];",
     "o[i] = y[i] * c[i] - y[i ^ 1] * s[i];"),
    ("rope: previous position's table row", "const double* c = cos_t + (int64_t)pos * half;",
     "const double* c = cos_t + (int64_t)(pos > 0 ? pos - 1 : 0) * half;"),
    ("rmsnorm: eps outside the root", "sqrt(ss / (double)D + eps)", "(sqrt(ss / (double)D) + eps)"),
    ("rmsnorm: sum instead of mean", "sqrt(ss / (double)D + eps)", "sqrt(ss + eps)"),
    ("rmsnorm: weight dropped", "y[d] = y[d] / r * half_bits_to_double(weight[d]);", "y[d] = y[d] / r;"),
    ("interleaved rope: sine sign flipped", "out[row + 2 * j] = u0 * c - u1 * sn;", "out[row + 2 * j] = u0 * c + u1 * sn;"),
    ("interleaved rope: position off by one", "const double ang = (double)t * pow(base, -2.0 * (double)j / (double)D);",
     "const double ang = (double)(t + 1) * pow(base, -2.0 * (double)j / (double)D);"),
    ("module: NeoX pairs instead of adjacent ones", "const double a = u[2 * j], b = u[2 * j + 1];",
     "const double a = u[j], b = u[j + D / 2];"),
    ("module: x W instead of x W^T", "half_bits_to_double(w_q[(int64_t)c * dim + e])",
     "half_bits_to_double(w_q[(int64_t)e * dim + c])"),
    ("module: key positions shifted by one", "const double pos = (double)(r % T);",
     "const double pos = (double)(r % T + which);"),
    ("module: scale 1/D", "const double scale = pow((double)D, -0.5);", "const double scale = pow((double)D, -1.0);"),
    ("module: output projection skipped", "out[r * dim + c] = s;", "out[r * dim + c] = A[r * dim + c];"),
    ("module: value projection with W_k", "sv += xe * half_bits_to_double(w_v[(int64_t)c * dim + e]);",
     "sv += xe * half_bits_to_double(w_k[(int64_t)c * dim + e]);"),
    ("rmsnorm: weight reversed", "y[d] = y[d] / r * half_bits_to_double(weight[d]);",
     "y[d] = y[d] / r * half_bits_to_double(weight[D - 1 - d]);"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, desc, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    path_c = tmp_path / "mutant.c"
    path_c.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    flags = obuild.cflags(sanitize=obuild.sanitize_requested(), opt="-O1")
    subprocess.run(["gcc"] + flags + ["-w", "-o", str(lib), str(path_c), "-lm"], check=True)
    ora = oracle.Oracle(str(lib))
    failed = []
    for pin in ALL_PINS:
        try:
            pin(ora)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake: {desc}"
