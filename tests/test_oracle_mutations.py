"""The oracle's pins must catch plausible mistakes.  Each case plants one
mistake in a copy of the oracle's C source (on the CPU only), builds it into
a temporary library and runs the pin suite against it in a subprocess; the
suite has to fail for every mutant."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "shrink_A_index_swapped": (
        "const float *ar = A[sig] + ((int64_t)s * R + j) * K;",
        "const float *ar = A[sig] + ((int64_t)j * L + s) * K;"),
    "shrink_drops_last_term": (
        "for (int32_t i = 0; i < K; ++i) acc = acc + xr[i] * ar[i];",
        "for (int32_t i = 0; i < K - 1; ++i) acc = acc + xr[i] * ar[i];"),
    "expand_B_transposed": (
        "const float *br = B[sig] + ((int64_t)s * N[sig] + n) * R;\n"
        "                float d = 0.0f;\n"
        "                for (int32_t j = 0; j < r; ++j) d = d + b[j] * br[j];",
        "const float *br = B[sig] + ((int64_t)s * N[sig]) * R + n;\n"
        "                float d = 0.0f;\n"
        "                for (int32_t j = 0; j < r; ++j) d = d + b[j] * br[j * N[sig]];"),
    "expand_scale_dropped": (
        "yr[off + n] = yr[off + n] + scale[s] * d;",
        "yr[off + n] = yr[off + n] + d;"),
    "expand_sign_flipped": (
        "yr[off + n] = yr[off + n] + scale[s] * d;",
        "yr[off + n] = yr[off + n] - scale[s] * d;"),
    "slice_offset_not_advanced": (
        "            off += N[sig];\n        }\n    }\n}\n\n/*\n * Packed apply",
        "        }\n    }\n}\n\n/*\n * Packed apply"),
    "rank_ignored": (
        "    if (r > R) r = R;",
        "    r = R;"),
    "rank0_slot_not_skipped": (
        "    if (r <= 0) return -1;",
        "    if (r < 0) return -1;"),
    "segments_unstable": (
        "        for (int32_t t = 0; t < T; ++t) {\n            int32_t r;\n            if (slot_of(idx, slot_rank, L, R, t, &r) == s) perm[pos++] = t;",
        "        for (int32_t t = T - 1; t >= 0; --t) {\n            int32_t r;\n            if (slot_of(idx, slot_rank, L, R, t, &r) == s) perm[pos++] = t;"),
    "moe_align_no_padding": (
        "                    while (pos % block_m) so[pos++] = P;",
        "                    ;"),
    "moe_shared_b_not_pinned": (
        "            int32_t eb = (E_b == 1) ? 0 : e;",
        "            int32_t eb = 0;"),
    "moe_weight_dropped": (
        "            if (kind == 1 && topk_w) coef = coef * topk_w[p];",
        "            ;"),
    "moe_w2_reads_token_row": (
        "            const float *xr = x + (kind == 0 ? t : p) * ldx;",
        "            const float *xr = x + (kind == 0 ? t : t) * ldx;"),
    "moe_expert_ignored_for_b": (
        "            int32_t eb = (E_b == 1) ? 0 : e;",
        "            int32_t eb = (E_b == 1) ? 0 : 0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(before, after, 1)
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "m.c")
        so = os.path.join(d, "libm.so")
        open(c, "w").write(mutated)
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                               "-std=c11", "-o", so, c])
        env = dict(os.environ, ADAPTER_APPLY_ORACLE_LIB=so)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
