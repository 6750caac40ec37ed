"""The oracle's pins are strong enough: plant one plausible mistake at a time
in a copy of the oracle's C source (a wrong index, a dropped term, a flipped
sign, a transposed operand, a wrong rounding tie), build it, run the pin
tests against it, and require that every mutant fails at least one pin.

The arithmetic of the fused K and V form on an fp8 cache is put together in
the oracle's Python layer, so its mutants are planted in a copy of that
module's source and run against the two V-leg pins directly."""
import importlib.util
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mla_oracle.c")
PINS = ["tests/test_oracle_codecs.py", "tests/test_oracle_gather.py",
        "tests/test_oracle_products.py", "tests/test_oracle_kv.py", "tests/test_oracle_latent_write.py",
        "tests/test_oracle_latent_write_fp8.py"]

MUTANTS = {
    "slot_uses_page_index": ("(p % P->page_size) * P->stride_token", "(p / P->page_size) * P->stride_token"),
    "layer_term_dropped": ("(int64_t)layer * P->stride_layer +", ""),
    "gather_start_off_by_one": ("token_offset(&P, b, (int64_t)cache_offsets[b] + i, layer, 0)",
                                "token_offset(&P, b, (int64_t)cache_offsets[b] + i + 1, layer, 0)"),
    "weight_transposed": ("elem(W, w_dtype, n * ldw + k)", "elem(W, w_dtype, k * ldw + n)"),
    "product_sign": ("s += elem(A, a_dtype, r * lda + k)", "s -= elem(A, a_dtype, r * lda + k)"),
    "last_k_dropped": ("for (int64_t k = 0; k < K; ++k)\n                s += elem",
                       "for (int64_t k = 0; k < K - 1; ++k)\n                s += elem"),
    "tie_to_odd": ("code = (lo & 1) ? hi : lo;", "code = (lo & 1) ? lo : hi;"),
    "subnormal_exponent": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    "bf16_shift": ("(uint32_t)h << 16", "(uint32_t)h << 15"),
    "inverse_scale_swapped": ("inv = 448.0f / amax;", "inv = amax / 448.0f;"),
    "act_scale_block_dropped": ("(double)sa[r * nkb + kb]", "(double)sa[r * nkb]"),
    "weight_scale_transposed": ("sw[(n / n_gran) * nkb + kb]", "sw[kb * nkb + (n / n_gran)]"),
    "no_saturation": ("if (a >= 448.0)\n        return sign | 0x7E;", "if (a > 464.0)\n        return 0x7F;"),
    "kv_half_ignored": ("(int64_t)kv * P->stride_kv +", ""),
    "kv_position_not_relative": ("(int64_t)cache_lengths[b] + (t - (int64_t)input_row_offsets[b])",
                                 "(int64_t)cache_lengths[b] + t"),
    "nn_weight_transposed": ("bf16_to_float(W[k * ldw + n])", "bf16_to_float(W[n * ldw + k])"),
    "rms_eps_dropped": ("sqrt(ss / (double)K + eps)", "sqrt(ss / (double)K)"),
    "rms_mean_over_row": ("sqrt(ss / (double)K + eps)", "sqrt(ss / (double)D + eps)"),
    "rope_sign": ("y[K + 2 * j] = x0 * c - x1 * s;", "y[K + 2 * j] = x0 * c + x1 * s;"),
    "rope_pair_swapped": ("double c = freqs[pos[t] * R + 2 * j], s = freqs[pos[t] * R + 2 * j + 1];",
                          "double s = freqs[pos[t] * R + 2 * j], c = freqs[pos[t] * R + 2 * j + 1];"),
    "cache_block_scale_inverted": ("to_codes = 448.0f / amax;", "to_codes = amax / 448.0f;"),
    "cache_short_block_widened": ("k1 = k0 + gran < D ? k0 + gran : D;", "k1 = k0 + gran;"),
    "rope_row_of_token": ("double c = freqs[pos[t] * R + 2 * j], s = freqs[pos[t] * R + 2 * j + 1];",
                          "double c = freqs[t * R + 2 * j], s = freqs[t * R + 2 * j + 1];"),
}


def _run_mutant(name, tmpdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    path = os.path.join(tmpdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(tmpdir, f"lib_{name}.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", so, path, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, MLA_ORACLE_LIB_OVERRIDE=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:randomly", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda n: _run_mutant(n, str(tmp_path)), MUTANTS))
    survivors = [n for n, rc in results if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"


# mistakes in how the V leg of the fp8-cache fused form is assembled
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")
PY_MUTANTS = {
    "v_reads_w_k": ("v = fp8_matmul_nt(codes[:, :case_v.K], scales[:, :kb], case_v.weight_q, case_v.weight_scale,",
                    "v = fp8_matmul_nt(codes[:, :case_v.K], scales[:, :kb], case_k.weight_q, case_k.weight_scale,"),
    "v_scale_slice_shifted": ("v = fp8_matmul_nt(codes[:, :case_v.K], scales[:, :kb],",
                              "v = fp8_matmul_nt(codes[:, :case_v.K], scales[:, 1:kb + 1],"),
}


def _python_mutant(name):
    import oracle
    old, new = PY_MUTANTS[name]
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    spec = importlib.util.spec_from_loader(f"oracle_mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__file__ = oracle.__file__      # loads the same built C library
    exec(compile(src.replace(old, new), PY_SRC, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_v_leg_mistakes_fail_a_pin(name):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import test_oracle_fp8_cache as pins
    mod = _python_mutant(name)
    caught = 0
    for check in (pins.check_kv_each_projection_on_its_own_weight, pins.check_kv_selection_w_uv):
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught, f"python mutant {name} passed every V-leg pin"
