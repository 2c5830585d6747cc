"""Each plausible mistake, planted in a COPY of oracle.c compiled to a
temporary library, must be caught by at least one pin (CPU only).  The oracle
itself is never modified.  Each mutant runs in a child process, so a mutant
that corrupts memory (and is thereby caught) cannot take the test run down."""
import os
import subprocess
import sys

import pytest

import oracle
import oracle.build
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, [(old, new), ...]); each `old` must occur in oracle.c.
MUTANTS = [
    ("drop_scale", [("s[j] = scale * acc;", "s[j] = acc;"),
                    ("s[j - j0] = scale * acc;", "s[j - j0] = acc;")]),
    ("exp_sign", [("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);")]),
    ("causal_off_by_one", [("long last = i + (Nk - Nq);", "long last = i + (Nk - Nq) - 1;")]),
    ("causal_top_left", [("long last = i + (Nk - Nq);", "long last = i;")]),
    ("gqa_modulo", [("long hk = h / G;", "long hk = h % Hkv;")]),
    ("k_for_v", [("orow[c] += a * V[j * d + c];", "orow[c] += a * K[j * d + c];")]),
    ("q_dot_q", [("acc += qrow[c] * K[j * d + c];", "acc += qrow[c] * qrow[c];")]),
    ("lse_without_max", [("*lse_out = m + log(l);\n}\n\n/* One output row by the blockwise",
                          "*lse_out = log(l);\n}\n\n/* One output row by the blockwise")]),
    ("no_normalisation", [("s[j] /= l;", "s[j] /= 1.0;")]),
    ("no_max_subtraction", [("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
                            ("*lse_out = m + log(l);\n}\n\n/* One output row by the blockwise",
                             "*lse_out = log(l);\n}\n\n/* One output row by the blockwise")]),
    ("blockwise_no_rescale", [("l *= alpha;", "l *= 1.0;")]),
    ("decode_drops_last_row", [("direct_row(q + r * d, K, V, L,", "direct_row(q + r * d, K, V, L > 0 ? L - 1 : 0,")]),
    ("decode_no_clamp", [("if (L > Lmax)\n                L = Lmax;", "")]),
    ("decode_wrong_head", [("long b = r / Hq, h = r % Hq, hk = h / G;", "long b = r / Hq, h = r % Hq, hk = h % Hkv;")]),
    ("paged_row_offset", [("* (long)bs + j % bs) * d;", "* (long)bs + j / bs) * d;")]),
    ("paged_head_major", [("const long src = ((blk * Hkv + hk)", "const long src = ((hk * num_blocks + blk)")]),
    ("paged_block_index", [("block_table[b * (long)max_blocks + j / bs]", "block_table[b * (long)max_blocks + j % max_blocks]")]),
    ("paged_no_entry_clamp", [("if (blk > num_blocks - 1)\n                    blk = num_blocks - 1;", "")]),
    ("bwd_drop_row_term", [("double ds = a[j] * (dp[j] - D);", "double ds = a[j] * dp[j];")]),
    ("bwd_dk_no_scale", [("dK[j * d + c] += scale * ds * qrow[c];", "dK[j * d + c] += ds * qrow[c];")]),
    ("bwd_dv_uses_ds", [("dV[j * d + c] += a[j] * dorow[c];", "dV[j * d + c] += ds * dorow[c];")]),
    ("bwd_dp_uses_k", [("acc += dorow[c] * V[j * d + c];", "acc += dorow[c] * K[j * d + c];")]),
    ("bwd_dq_uses_v", [("dqrow[c] += scale * ds * K[j * d + c];", "dqrow[c] += scale * ds * V[j * d + c];")]),
    ("bwd_dq_sign", [("dqrow[c] += scale * ds * K[j * d + c];", "dqrow[c] -= scale * ds * K[j * d + c];")]),
    ("bwd_first_head_only", [("for (long h = hk * G; h < (hk + 1) * G; ++h) { /* [E] sec. 2.3 */",
                              "for (long h = hk * G; h < hk * G + 1; ++h) {")]),
    ("bwd_unmasked", [("visible_keys(i, Nq, Nk, causal), d, scale, a, dp,", "Nk, d, scale, a, dp,")]),
    ("bwd_rows_weight_without_lse", [("const double aij = exp(scale * s - lse[r]);",
                                      "const double aij = exp(scale * s);")]),
    ("bwd_rows_no_row_term", [("Dst[r] = D;", "Dst[r] = 0.0;")]),
    ("bwd_rows_sees_future", [("if (j >= visible_keys(i, Nq, Nk, causal))", "if (j >= Nk)")]),
]


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, "mutation site not found: %r" % old
        src = src.replace(old, new)
    msrc = tmp_path / ("oracle_%s.c" % name)
    msrc.write_text(src)
    lib = oracle.build.build(src=str(msrc), out=str(tmp_path / ("liboracle_%s.so" % name)))
    here = os.path.dirname(os.path.abspath(__file__))
    code = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import oracle, oracle_pins as P\n"
        "mut = oracle.Oracle(%r)\n"
        "caught = []\n"
        "for pin in P.ALL_PINS:\n"
        "    try:\n"
        "        pin(mut)\n"
        "    except Exception as e:\n"
        "        caught.append(pin.__name__)\n"
        "print('CAUGHT', ','.join(caught))\n"
    ) % (here, os.path.dirname(here), lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, OMP_NUM_THREADS="2"))
    if r.returncode != 0:
        return  # the mutant crashed the process: caught
    line = [x for x in r.stdout.splitlines() if x.startswith("CAUGHT")][-1]
    caught = [x for x in line.split(" ", 1)[1].split(",") if x] if " " in line else []
    assert caught, "mutant %s passed every pin" % name
