"""Planted-mistake check of the oracle's pins (CPU only; not collected by
pytest: run it as ``python tests/oracle_mutations.py``).

Each entry below is a plausible mistake in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a misread of the pages).  For
each, the oracle sources are copied to a temporary tree with the mistake
planted, the oracle's C library is rebuilt there, and the oracle's pin
tests (tests/test_oracle*.py, which run on the CPU) are run against it.
Every mistake must make at least one pin fail; the script exits non-zero if
one survives.  tests/test_oracle.py checks on every CPU run that each
mistake still applies to the current sources, so this list stays runnable.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C = "oracle/sink_attn_oracle.c"
ROPE = "oracle/rope.py"

# (name, file, text to find -- exactly once --, replacement)
MUTATIONS = [
    # the definition of the sink-aware softmax
    ("sink dropped from the denominator", C,
     "double Z = exp(sigma - M);", "double Z = 0.0;"),
    ("sink scaled by the softmax scale", C,
     "(double)c->sinks[h] : -INFINITY;", "(double)c->sinks[h] * c->sm_scale : -INFINITY;"),
    ("sink carries the first key's value", C,
     "  if (w_sink) *w_sink = exp(sigma - M) / Z;\n",
     "  if (j1 > j0) {\n    const uint16_t* v0 = c->v + kv_row_offset(c, b, j0, g);\n"
     "    for (int x = 0; x < D; ++x) o[x] += exp(sigma - M) / Z * bf16_to_double(v0[x]);\n  }\n"
     "  if (w_sink) *w_sink = exp(sigma - M) / Z;\n"),
    ("GQA map h mod Hkv", C, "const int g = h / G;", "const int g = h % c->hkv;"),
    ("causal limit off by one", C,
     "hi = p + 1 < L ? p + 1 : L;", "hi = p < L ? p : L;"),
    ("top-left causal alignment", C,
     "int64_t p = L - qlen + t;  /* absolute position of the query */",
     "int64_t p = t;  /* absolute position of the query */"),
    ("wrong page slot", C,
     "int64_t slot = j % c->page_size;", "int64_t slot = (j + 1) % c->page_size;"),
    ("page table offset missing", C,
     "c->page_indices[(int64_t)c->kv_indptr[b] + j / c->page_size];",
     "c->page_indices[j / c->page_size];"),
    ("sink in every partial", C,
     "(c->include_sink && c->sinks) ?", "(c->sinks) ?"),
    ("lse without the maximum", C, "*lse = M + log(Z);", "*lse = log(Z);"),
    ("contiguous K/V head-major", C,
     "return (tok * c->hkv + g) * c->d;", "return (tok + (int64_t)g * c->hkv) * c->d;"),
    ("merge weight sign flipped", C, "else w = exp(ls[s] - L);", "else w = exp(L - ls[s]);"),
    ("merge lse without the log", C,
     "lse[i] = (L == INFINITY) ? INFINITY : L + log(W);",
     "lse[i] = (L == INFINITY) ? INFINITY : L + W;"),
    ("softmax scale dropped", C, "double s = c->sm_scale * dot;", "double s = dot;"),
    ("half of the dot product", C,
     "for (int x = 0; x < D; ++x) dot += ", "for (int x = 0; x < D / 2; ++x) dot += "),
    ("weights normalised without the sink", C,
     "double p = exp(scores[j - j0] - M) / Z;",
     "double p = exp(scores[j - j0] - M) / (Z - exp(sigma - M));"),
    # the draft (tree) mask
    ("draft bit index off by one", C,
     "return (int)((c->draft_mask[row] >> i) & 1u);",
     "return (int)((c->draft_mask[row] >> (i + 1)) & 1u);"),
    ("draft mask transposed", C,
     "return (int)((c->draft_mask[row] >> i) & 1u);",
     "return (int)((c->draft_mask[c->qo_indptr[b] + i] >> (row - c->qo_indptr[b])) & 1u);"),
    ("prefix hidden under a draft mask", C,
     "if (i < 0) return 1;        /* a prefix key */", "if (i < 0) return 0;        /* a prefix key */"),
    ("causality kept under a draft mask", C,
     "if (c->causal && !c->draft_mask) {", "if (c->causal) {"),
    ("masked drafted keys still scored", C,
     "if (!key_allowed(c, b, row, j)) { scores[j - j0] = -INFINITY; continue; }",
     "if (0) { scores[j - j0] = -INFINITY; continue; }"),
    # bias, YaRN rotary encoding and the paged append
    ("bias after the rotation", ROPE,
     "q[row, h] = rotate(qkv[row, h] + bias[h], cos, sin, interleaved)",
     "q[row, h] = rotate(qkv[row, h], cos, sin, interleaved) + bias[h]"),
    ("rotation sign", ROPE,
     "y[i] = x[i] * cos[d] - x[j] * sin[d]", "y[i] = x[i] * cos[d] + x[j] * sin[d]"),
    ("YaRN ramp bounds swapped", ROPE,
     "gamma = (r - beta_slow) / (beta_fast - beta_slow)",
     "gamma = (r - beta_fast) / (beta_slow - beta_fast)"),
    ("wavelength without 2 pi", ROPE,
     "wavelength = 2.0 * math.pi / theta", "wavelength = 1.0 / theta"),
    ("YaRN scale applied the wrong way", ROPE,
     "out[d] = (1.0 - gamma) * theta / factor + gamma * theta",
     "out[d] = (1.0 - gamma) * theta * factor + gamma * theta"),
    ("no attention temperature", ROPE,
     "return 0.1 * math.log(factor) + 1.0 if factor > 1.0 else 1.0", "return 1.0"),
    ("append position off by one", ROPE,
     "p = int(kv_len[b]) - qlen + t", "p = int(kv_len[b]) - qlen + t + 1"),
    ("rotated pairings swapped", ROPE, "    if interleaved:\n", "    if not interleaved:\n"),
    ("frequency exponent halved", ROPE,
     "theta = base ** (-2.0 * d / head_dim)", "theta = base ** (-1.0 * d / head_dim)"),
    ("pair ramp bounds rounded the wrong way", ROPE,
     "low = max(math.floor(correction_pair(beta_fast, head_dim, base, original_max_pos)), 0)",
     "low = max(math.ceil(correction_pair(beta_fast, head_dim, base, original_max_pos)), 0)"),
    ("pair ramp blended the wrong way", ROPE,
     "gamma = min(max(1.0 - (d - low) / (high - low), 0.0), 1.0)",
     "gamma = min(max((d - low) / (high - low), 0.0), 1.0)"),
    ("append to the page of the next position", ROPE,
     "page = int(page_indices[int(page_indptr[b]) + p // page_size])",
     "page = int(page_indices[int(page_indptr[b]) + (p + 1) // page_size])"),
]

PIN_TESTS = ["tests/test_oracle.py", "tests/test_oracle_draft_mask.py", "tests/test_oracle_rope.py"]
COPY = ["oracle", "tests", "workloads", "gqa_attention_sinks_attn_amd", "include"]


def plant(text: str, find: str, replace: str) -> str:
    if text.count(find) != 1:
        raise ValueError(f"expected exactly one occurrence of {find!r}, found {text.count(find)}")
    return text.replace(find, replace)


def check_applicable():
    """Every mistake still applies to the current sources (used by the CPU tests)."""
    for name, path, find, replace in MUTATIONS:
        with open(os.path.join(ROOT, path)) as f:
            plant(f.read(), find, replace)


def run_one(name, path, find, replace) -> bool:
    """True when the planted mistake makes a pin fail."""
    with tempfile.TemporaryDirectory(prefix="oracle_mut_") as tmp:
        for d in COPY:
            shutil.copytree(os.path.join(ROOT, d), os.path.join(tmp, d),
                            ignore=shutil.ignore_patterns("__pycache__", "libsink_attn_oracle.so",
                                                          "*.tmp*"))
        dst = os.path.join(tmp, path)
        with open(dst) as f:
            text = f.read()
        with open(dst, "w") as f:
            f.write(plant(text, find, replace))
        env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            "-m", "not gpu", *PIN_TESTS], cwd=tmp, env=env,
                           capture_output=True, text=True, timeout=900)
        return r.returncode != 0


def main() -> int:
    check_applicable()
    survivors = []
    for name, path, find, replace in MUTATIONS:
        caught = run_one(name, path, find, replace)
        print(f"{'caught ' if caught else 'SURVIVED'}  {name}  ({path})", flush=True)
        if not caught:
            survivors.append(name)
    print(f"{len(MUTATIONS) - len(survivors)} of {len(MUTATIONS)} planted mistakes caught", flush=True)
    return 1 if survivors else 0


if __name__ == "__main__":
    sys.exit(main())
