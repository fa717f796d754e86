"""Oracle of the step that feeds the attention path: QKV bias, YaRN rotary
position encoding and the append of the new keys and values to the paged
cache.  fp64, numpy, plain loops over tokens.  TEST INFRASTRUCTURE ONLY:
only the tests, the smoke check and the benchmark's CPU-baseline leg may
import it; it shares no code with the GPU library.

What the pages fix, and the readings taken where they stop:

* "GPT-OSS on Day 0" (Perplexity), section "Attention: GQA with attention
  sinks": the model encodes positions with YaRN "like DeepSeek-V3" and its
  QKV projections carry a bias "like Qwen 2".  No formula or constant is
  given.  Readings:
  - the bias is part of the projection, so it is added before the rotation;
    the value heads get the bias and no rotation;
  - YaRN is taken as published (Peng et al., "YaRN: Efficient Context Window
    Extension of Large Language Models", 2023): rotary frequencies
    theta_d = base^(-2d/D) for pair d < D/2; wavelength lambda_d =
    2 pi / theta_d; r_d = L / lambda_d with L the original context length;
    ramp gamma(r) = 0 for r < alpha, 1 for r > beta, (r - alpha) / (beta -
    alpha) between ("NTK-by-parts"); new frequency
    (1 - gamma) theta_d / s + gamma theta_d for scale factor s; and the
    attention temperature sqrt(1/t) = 0.1 ln s + 1 applied to both q and k,
    i.e. to every cos and sin.  s <= 1 is plain rotary encoding (no change,
    temperature 1).  base, s, L, alpha (beta_slow) and beta (beta_fast) are
    parameters;
  - "like DeepSeek-V3": DeepSeek-V3 (and the YaRN authors' released code)
    blend linearly in the pair index instead of the rotation count: the
    pair d at which the wavelength fits r turns in L is d(r) = D ln(L /
    (2 pi r)) / (2 ln base); with low = floor(d(beta)) and high =
    ceil(d(alpha)) (clamped to the pairs that exist), gamma(d) = 1 - (d -
    low) / (high - low), clamped to [0, 1] (a step at low when high <= low).
    Both ramps are offered ("turns", the published formula, and "pairs");
    they agree on which pairs keep, ramp or divide by s, and differ in the
    blend of the ramped pairs;
  - pairing: the pages do not say which dimensions form a rotated pair.
    "half" rotates dimension i with i + D/2 (the rotate-half layout),
    "interleaved" rotates 2i with 2i + 1 (the complex-pair layout); both
    are offered.
* "Accelerating Sonar Through Speculation" (Perplexity), section "Inference
  with Speculative Decoding": before a step runs, the scheduler reserves
  room for the next tokens in the paged KV cache and ships the page
  information with the batch.  Reading: the new tokens of request b are the
  last qlen_b positions of its kv_len_b keys (the alignment the attention
  path uses), token t sits at p = kv_len_b - qlen_b + t, and its key and
  value go to slot p % page_size of page page_indices[page_indptr[b] +
  p // page_size].  Every other slot of the cache is left as it was.

Layouts (the library's):
  qkv      bf16 bits [T, Hq + 2 Hkv, D]: query heads, then key heads, then
           value heads of each new token;  bias bf16 bits [(Hq + 2 Hkv) D]
  table    [max_pos, D]: cos of pair d times the temperature in column d,
           sin times the temperature in column D/2 + d
  pages    bf16 bits [num_pages, Hkv, page_size, D]
"""
from __future__ import annotations

import math

import numpy as np


def _bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)) \
        .view(np.float32).astype(np.float64)


def correction_pair(rotations: float, head_dim: int, base: float, original_max_pos: int) -> float:
    """The fractional pair index whose wavelength 2 pi base^(2d/D) fits
    `rotations` turns in the original context."""
    return head_dim * math.log(original_max_pos / (2.0 * math.pi * rotations)) / (2.0 * math.log(base))


def yarn_frequencies(head_dim: int, base: float, factor: float, original_max_pos: int,
                     beta_fast: float, beta_slow: float, ramp: str = "turns") -> np.ndarray:
    """Rotary frequency of each of the head_dim / 2 pairs (YaRN, NTK-by-parts).
    ramp: "turns" blends linearly in the rotation count, "pairs" linearly in
    the pair index between the rounded correction pairs."""
    if ramp not in ("turns", "pairs"):
        raise ValueError(ramp)
    half = head_dim // 2
    out = np.zeros(half)
    if ramp == "pairs" and factor > 1.0:
        low = max(math.floor(correction_pair(beta_fast, head_dim, base, original_max_pos)), 0)
        high = min(math.ceil(correction_pair(beta_slow, head_dim, base, original_max_pos)), half - 1)
    for d in range(half):
        theta = base ** (-2.0 * d / head_dim)
        if factor <= 1.0:
            out[d] = theta
            continue
        if ramp == "pairs":
            if high <= low:
                gamma = 1.0 if d <= low else 0.0
            else:
                gamma = min(max(1.0 - (d - low) / (high - low), 0.0), 1.0)
        else:
            wavelength = 2.0 * math.pi / theta
            r = original_max_pos / wavelength      # rotations within the original context
            if r < beta_slow:
                gamma = 0.0                        # long wavelengths: interpolate fully
            elif r > beta_fast:
                gamma = 1.0                        # short wavelengths: keep
            else:
                gamma = (r - beta_slow) / (beta_fast - beta_slow)
        out[d] = (1.0 - gamma) * theta / factor + gamma * theta
    return out


def yarn_temperature(factor: float) -> float:
    """sqrt(1/t): the factor YaRN applies to q and k (so to every cos, sin)."""
    return 0.1 * math.log(factor) + 1.0 if factor > 1.0 else 1.0


def rope_table(max_pos: int, head_dim: int, base: float, factor: float, original_max_pos: int,
               beta_fast: float, beta_slow: float, attn_factor: float = 0.0,
               ramp: str = "turns") -> np.ndarray:
    """[max_pos, head_dim]: temperature * cos(p f_d) in column d, temperature *
    sin(p f_d) in column head_dim/2 + d.  attn_factor <= 0: YaRN's own."""
    f = yarn_frequencies(head_dim, base, factor, original_max_pos, beta_fast, beta_slow, ramp)
    m = attn_factor if attn_factor > 0 else yarn_temperature(factor)
    half = head_dim // 2
    tab = np.zeros((max_pos, head_dim))
    for p in range(max_pos):
        for d in range(half):
            tab[p, d] = m * math.cos(p * f[d])
            tab[p, half + d] = m * math.sin(p * f[d])
    return tab


def _pairs(head_dim: int, interleaved: bool):
    """(first, second) dimension of each rotated pair d."""
    half = head_dim // 2
    if interleaved:
        return [(2 * d, 2 * d + 1) for d in range(half)]
    return [(d, d + half) for d in range(half)]


def rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, interleaved: bool) -> np.ndarray:
    """Rotate each pair (a, b) of x [D] by the angle whose cos and sin (already
    times the temperature) are given per pair: (a c - b s, b c + a s)."""
    y = np.array(x, dtype=np.float64)
    for d, (i, j) in enumerate(_pairs(x.shape[0], interleaved)):
        y[i] = x[i] * cos[d] - x[j] * sin[d]
        y[j] = x[j] * cos[d] + x[i] * sin[d]
    return y


def qkv_rope_append(qkv_bits, bias_bits, table, qo_indptr, kv_len, page_indptr, page_indices,
                    k_pages_bits, v_pages_bits, hq: int, hkv: int, interleaved: bool,
                    rows=None):
    """Returns (q [T, Hq, D], k_cache, v_cache) in fp64.  The caches are the
    input caches (widened) with the new tokens' slots replaced by their
    biased, rotated keys and biased values.  Each request's positions must lie
    inside the table and its reserved pages.  rows: evaluate only these token
    rows (the others stay 0 in q and untouched in the caches)."""
    wanted = None if rows is None else set(int(r) for r in rows)
    qkv = _bf16_to_f64(qkv_bits)
    T, H, D = qkv.shape
    assert H == hq + 2 * hkv
    bias = np.zeros((H, D)) if bias_bits is None else _bf16_to_f64(bias_bits).reshape(H, D)
    kc = _bf16_to_f64(k_pages_bits).copy()
    vc = _bf16_to_f64(v_pages_bits).copy()
    page_size = kc.shape[2]
    half = D // 2
    q = np.zeros((T, hq, D))
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        qlen = q1 - q0
        for t in range(qlen):
            row = q0 + t
            if wanted is not None and row not in wanted:
                continue
            p = int(kv_len[b]) - qlen + t
            assert 0 <= p < table.shape[0]
            cos, sin = table[p, :half], table[p, half:]
            page = int(page_indices[int(page_indptr[b]) + p // page_size])
            slot = p % page_size
            for h in range(hq):
                q[row, h] = rotate(qkv[row, h] + bias[h], cos, sin, interleaved)
            for g in range(hkv):
                kc[page, g, slot] = rotate(qkv[row, hq + g] + bias[hq + g], cos, sin, interleaved)
                vc[page, g, slot] = qkv[row, hq + hkv + g] + bias[hq + hkv + g]
    return q, kc, vc
