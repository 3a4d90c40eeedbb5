"""Mutation check of the oracle's pins, on the CPU.

Each case plants one plausible mistake (a dropped term, a wrong sign, index or
bound, a transposed operand) in a private copy of ``oracle/mimo_oracle.c``,
builds it with gcc into a temporary directory, runs the pins of
``oracle_pins`` against that build in a subprocess until one fails, and
requires that one does.  The planted source never leaves the temporary
directory.  The mutants are checked in parallel, a few processes at a time.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

MUTANTS = {
    "sink dropped from the denominator": ("    if (has_sink) z += exp(sigma - m);\n", "\n"),
    "sink given a value row (key 0)": (
        "    for (int e = 0; e < d->dv; ++e) o[e] *= d->value_scale;\n",
        "    if (has_sink) for (int e = 0; e < d->dv; ++e) o[e] += exp(sigma - l) * bf16_to_double(vrows[0][e]);\n"
        "    for (int e = 0; e < d->dv; ++e) o[e] *= d->value_scale;\n"),
    "sink scaled like a score": ("    *sigma = s;\n", "    *sigma = s * 0.0721687836;\n"),
    "window one key too wide (prefill)": (
        "        if (d->layer_type == ORACLE_SWA) lo = p - (d->window - 1) > 0 ? p - (d->window - 1) : 0;\n"
        "        for (int h = 0;",
        "        if (d->layer_type == ORACLE_SWA) lo = p - d->window > 0 ? p - d->window : 0;\n"
        "        for (int h = 0;"),
    "causal bound excludes self": ("    for (int j = lo; j <= p; ++j, ++n) {\n        kr[n] = k + ",
                                   "    for (int j = lo; j < p; ++j, ++n) {\n        kr[n] = k + "),
    "GQA heads interleaved instead of grouped": ("            int g = h / group;\n            int n = prefill_key_rows(",
                                                 "            int g = h % d->hkv;\n            int n = prefill_key_rows("),
    "wrong KV head for keys": (
        "        kr[n] = k + ((size_t)(base + j) * d->hkv + g) * d->dqk;\n",
        "        kr[n] = k + ((size_t)(base + j) * d->hkv + (g + 1) % d->hkv) * d->dqk;\n"),
    "value_scale not applied": ("    for (int e = 0; e < d->dv; ++e) o[e] *= d->value_scale;\n", "\n"),
    "softmax scale not applied": ("        scores[j] = d->scale * acc;\n", "        scores[j] = acc;\n"),
    "LSE without the max": ("    double l = m + log(z);\n", "    double l = log(z);\n"),
    "score sign flipped": ("        scores[j] = d->scale * acc;\n", "        scores[j] = -d->scale * acc;\n"),
    "weights not normalised by the sink": ("        double w = exp(scores[j] - l);\n",
                                           "        double w = exp(scores[j] - l) * (has_sink ? z / (z - exp(sigma - m)) : 1.0);\n"),
    "ring slot off by one (cache read)": (
        "    if (d->layer_type == ORACLE_SWA) row = (size_t)b * ring + (size_t)(j % ring);\n",
        "    if (d->layer_type == ORACLE_SWA) row = (size_t)b * ring + (size_t)((j + 1) % ring);\n"),
    "decode new token read from the cache": (
        "        kr[n] = jb->k_new + ((size_t)b * d->hkv + g) * d->dqk;\n",
        "        kr[n] = cache_row(jb, b, p > 0 ? p - 1 : 0, g, 0);\n"),
    "decode window one key too narrow": (
        "        if (d->layer_type == ORACLE_SWA) lo = p - (d->window - 1) > 0 ? p - (d->window - 1) : 0;\n"
        "        int n = 0;\n        for (int j = lo; j < p; ++j, ++n) {",
        "        if (d->layer_type == ORACLE_SWA) lo = p - (d->window - 2) > 0 ? p - (d->window - 2) : 0;\n"
        "        int n = 0;\n        for (int j = lo; j < p; ++j, ++n) {"),
    "chunk reads its first own key from the cache": ("            } else if (j < c) {\n", "            } else if (j <= c) {\n"),
    "FP8 chunk reads its cached codes one row late": (
        "/* FP8 codes of the GA pool row (contiguous or paged) */\n"
        "                size_t row = jb->pages ? (size_t)paged_row(jb->pages, b, j) : (size_t)(jb->kv_base[b] + j);\n",
        "/* FP8 codes of the GA pool row (contiguous or paged) */\n"
        "                size_t row = jb->pages ? (size_t)paged_row(jb->pages, b, j) : (size_t)(jb->kv_base[b] + j + 1);\n"),
    "FP8 chunk cached keys without the K scale": (
        "        fp8_rows_t f8 = {k8r, v8r, jb->f8 ? (double)jb->f8->kscale[g] : 1.0,",
        "        fp8_rows_t f8 = {k8r, v8r, 1.0,"),
    "FP8 paged append at the flat row": ("                dst = (size_t)paged_row(pages, b, pos);\n",
                                          "                dst = (size_t)pos;\n"),
    "FP8 paged append room one row short": (
        "        int64_t room = pages ? (int64_t)pages->max_blocks * pages->page_size : kv_capacity[b];\n",
        "        int64_t room = pages ? (int64_t)pages->max_blocks * pages->page_size - 1 : kv_capacity[b];\n"),
    "chunk query position without the cached offset": ("        int p = c + (int)(t - jb->cu[b]);\n",
                                                       "        int p = (int)(t - jb->cu[b]);\n"),
    "chunk window one key too wide": (
        "        if (d->layer_type == ORACLE_SWA) lo = p - (d->window - 1) > 0 ? p - (d->window - 1) : 0;\n"
        "        int n = 0;\n        for (int j = lo; j <= p; ++j, ++n) {",
        "        if (d->layer_type == ORACLE_SWA) lo = p - d->window > 0 ? p - d->window : 0;\n"
        "        int n = 0;\n        for (int j = lo; j <= p; ++j, ++n) {"),
    "append ring slot off by one": (
        "            size_t dst = layer_type == ORACLE_SWA ? (size_t)b * ring_slots + (size_t)(pos % ring_slots)\n",
        "            size_t dst = layer_type == ORACLE_SWA ? (size_t)b * ring_slots + (size_t)((pos + 1) % ring_slots)\n"),
    "ring reader hard-coded to 128 slots": (
        "    if (d->layer_type == ORACLE_SWA) row = (size_t)b * ring + (size_t)(j % ring);\n",
        "    if (d->layer_type == ORACLE_SWA) row = (size_t)b * ring + (size_t)(j % 128);\n"),
    "ring append hard-coded to 128 slots": (
        "            size_t dst = layer_type == ORACLE_SWA ? (size_t)b * ring_slots + (size_t)(pos % ring_slots)\n",
        "            size_t dst = layer_type == ORACLE_SWA ? (size_t)b * ring_slots + (size_t)(pos % 128)\n"),
    "append capacity check off by one": ("        if (layer_type == ORACLE_GA && (int64_t)ctx_lens[b] + n > kv_capacity[b]) {\n",
                                         "        if (layer_type == ORACLE_GA && (int64_t)ctx_lens[b] + n >= kv_capacity[b]) {\n"),
    "paged row inside the page from the block index": (
        "    return page * pg->page_size + j % pg->page_size;\n",
        "    return page * pg->page_size + (j / pg->page_size) % pg->page_size;\n"),
    "paged block table rows strided by the page size": (
        "    int64_t page = pg->table[(size_t)b * pg->max_blocks + (size_t)(j / pg->page_size)];\n",
        "    int64_t page = pg->table[(size_t)b * pg->page_size + (size_t)(j / pg->page_size)];\n"),
    "paged append capacity check off by one": (
        "        if ((int64_t)ctx_lens[b] + n > (int64_t)max_blocks * page_size) {\n",
        "        if ((int64_t)ctx_lens[b] + n >= (int64_t)max_blocks * page_size) {\n"),
    "paged append writes tokens on unmapped blocks": (
        "            if (page < 0 || page >= num_pages) {\n                status = ORACLE_ECAPACITY;\n                continue;\n            }\n",
        "            if (page >= num_pages) {\n                status = ORACLE_ECAPACITY;\n                continue;\n            }\n"),
    "E4M3 rounds half away from zero": ("    double step = ldexp(1.0, b - 3);\n    double r = nearbyint(a / step) * step;",
                                        "    double step = ldexp(1.0, b - 3);\n    double r = round(a / step) * step;"),
    "E4M3 not saturated at 448": ("    if (a > 448.0) a = 448.0;\n", "\n"),
    "E4M3 subnormal step one binade off": ("    int b = -6;\n", "    int b = -7;\n"),
    "E4M3 decode exponent bias off by one": ("    return sgn * ldexp(1.0 + (double)m / 8.0, e - 7);\n",
                                             "    return sgn * ldexp(1.0 + (double)m / 8.0, e - 8);\n"),
    "FP8 decode ignores the K scale": (
        "                acc += bf16_to_double(qrow[x]) * (e4m3_to_double(f8->k8[j][x]) * f8->kscale);\n",
        "                acc += bf16_to_double(qrow[x]) * e4m3_to_double(f8->k8[j][x]);\n"),
    "FP8 decode applies the K scale to values": (
        "            for (int e = 0; e < d->dv; ++e) o[e] += w * (e4m3_to_double(f8->v8[j][e]) * f8->vscale);\n",
        "            for (int e = 0; e < d->dv; ++e) o[e] += w * (e4m3_to_double(f8->v8[j][e]) * f8->kscale);\n"),
    "FP8 append uses head 0's scale": (
        "                    k_cache[(dst * hkv + g) * dqk + x] = e4m3_quantize(k[(src * hkv + g) * dqk + x], k_scale[g]);\n",
        "                    k_cache[(dst * hkv + g) * dqk + x] = e4m3_quantize(k[(src * hkv + g) * dqk + x], k_scale[0]);\n"),
    "FP8 quantiser multiplies by the scale": ("    return e4m3_from_float(f / scale);\n", "    return e4m3_from_float(f * scale);\n"),
    "backward dS without the D term (dq)": ("                    double ds = w[j] * (d->value_scale * dp - D);\n",
                                            "                    double ds = w[j] * (d->value_scale * dp);\n"),
    "backward dS without value_scale (dk)": (
        "                        double ds = pw * (d->value_scale * dp - jb->D[row]);\n",
        "                        double ds = pw * (dp - jb->D[row]);\n"),
    "backward dv without value_scale": (
        "                        for (int e = 0; e < d->dv; ++e) dv[e] += d->value_scale * pw * bf16_to_double(dorow[e]);\n",
        "                        for (int e = 0; e < d->dv; ++e) dv[e] += pw * bf16_to_double(dorow[e]);\n"),
    "backward dk without the softmax scale": (
        "                        for (int x = 0; x < d->dqk; ++x) dk[x] += d->scale * ds * bf16_to_double(qrow[x]);\n",
        "                        for (int x = 0; x < d->dqk; ++x) dk[x] += ds * bf16_to_double(qrow[x]);\n"),
    "backward dsink sign flipped": ("            for (int64_t r = 0; r < T; ++r) acc -= ps[(size_t)r * hq + h] * D[(size_t)r * hq + h];\n",
                                    "            for (int64_t r = 0; r < T; ++r) acc += ps[(size_t)r * hq + h] * D[(size_t)r * hq + h];\n"),
    "backward SWA receivers one too many": (
        "            if (d->layer_type == ORACLE_SWA && p + d->window - 1 < hi) hi = p + d->window - 1;\n",
        "            if (d->layer_type == ORACLE_SWA && p + d->window < hi) hi = p + d->window;\n"),
    "backward D from the value instead of the output": (
        "                    D += bf16_to_double(dorow[e]) * (jb->stored_out ? round_bf16(o[e]) : o[e]);\n",
        "                    D += bf16_to_double(dorow[e]) * (jb->stored_out ? round_bf16(o[e]) : o[e]) / d->value_scale;\n"),
    "backward stored output left unrounded": ("(jb->stored_out ? round_bf16(o[e]) : o[e])", "o[e]"),
    "bf16 rounding truncates": ("    double step = ldexp(1.0, b - 7);\n    double r = nearbyint(a / step) * step;",
                                "    double step = ldexp(1.0, b - 7);\n    double r = floor(a / step) * step;"),
    "bf16 rounding keeps one bit too few": ("    double step = ldexp(1.0, b - 7);\n", "    double step = ldexp(1.0, b - 6);\n"),
    "rope pairs neighbours instead of halves": ("        double a = bf16_to_double(x[i]), b = bf16_to_double(x[i + half]);\n",
                                                "        double a = bf16_to_double(x[i]), b = bf16_to_double(x[(i ^ 1)]);\n"),
    "rope rotates the wrong way": ("        out[i] = a * c - b * sn;\n", "        out[i] = a * c + b * sn;\n"),
    "rope frequencies over the head dim": ("        double f = pow(theta, -2.0 * i / rd);\n",
                                           "        double f = pow(theta, -2.0 * i / d);\n"),
    "bf16 widened from the wrong half": ("    uint32_t w = ((uint32_t)bits) << 16;\n", "    uint32_t w = ((uint32_t)bits) << 15;\n"),
}


def _run_mutant(name, workdir):
    """Build the oracle with one planted mistake and run the pins against it until
    one fails.  Returns (caught, report)."""
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    if src.count(old) != 1:
        return False, f"mutation site for '{name}' not found exactly once"
    mpath = os.path.join(workdir, "mutant.c")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(workdir, "libmutant.so")
    oracle.build(mpath, lib)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib, "--first"],
                         capture_output=True, text=True, timeout=600, env=env)
    lines = [l for l in res.stdout.splitlines() if l.startswith("FAILED:")]
    # A crash of the planted build also counts as caught, but only a clean run
    # that names a failing pin tells which pin caught it.
    caught = (res.returncode != 0) or bool(lines and lines[-1] != "FAILED:")
    return caught, f"{res.stdout[-2000:]}\n{res.stderr[-2000:]}"


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Every mutant, built and checked in parallel (each check is its own process)."""
    workers = max(1, min(4, (os.cpu_count() or 2) // 2))
    dirs = {name: str(tmp_path_factory.mktemp("mutant")) for name in MUTANTS}
    with ThreadPoolExecutor(workers) as pool:
        futures = {name: pool.submit(_run_mutant, name, dirs[name]) for name in MUTANTS}
        return {name: f.result() for name, f in futures.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, mutant_results):
    caught, report = mutant_results[name]
    assert caught, f"no pin caught mutant '{name}'\n{report}"
