"""The pins must catch plausible mistakes in the oracle.

Each case plants one error in a copy of oracle/rt_oracle.c (or, where a third
item names it, another file of the oracle) on the CPU, in a temporary
directory, rebuilds it, and runs tests/test_oracle_pins.py against the copy: at
least one pin has to fail.  The unmodified copy has to pass.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle")

MUTANTS = {
    "self_not_visible": ("ok[s] = (!causal) || (p[s] <= p[r]);",
                         "ok[s] = (!causal) || (p[s] < p[r]);"),
    "tie_break_flipped": ("return (x->t < y->t) ? -1 : (x->t > y->t);\n}\n\nstatic int by_int",
                          "return (x->t > y->t) ? -1 : (x->t < y->t);\n}\n\nstatic int by_int"),
    "smallest_scores": ("*y = (const scored_t *)b;\n    if (x->s > y->s) return -1;\n"
                        "    if (x->s < y->s) return 1;",
                        "*y = (const scored_t *)b;\n    if (x->s < y->s) return -1;\n"
                        "    if (x->s > y->s) return 1;"),
    "no_normalisation": ("xhat[t * d + i] = x[t * d + i] / r;", "xhat[t * d + i] = x[t * d + i];"),
    "ema_missing_half": ("(1.0 - lam) * 0.5 * (sum_q[j] + sum_k[j])",
                         "(1.0 - lam) * (sum_q[j] + sum_k[j])"),
    "ema_wrong_weight": ("mu[j] = lam * mu[j]", "mu[j] = (1.0 - lam) * mu[j]"),
    "scatter_overwrites": ("out[t * d + i] += o[((long)c * w + r) * d + i];",
                           "out[t * d + i] = o[((long)c * w + r) * d + i];"),
    "scale_dropped": ("logit[s] = scale * dot;", "logit[s] = dot;"),
    "local_window_off_by_one": ("(size_t)(2 * window + 1));\n    for (long i = 0; i < n; ++i) {\n"
                                "        long lo = i - window + 1;\n        if (lo < 0)\n"
                                "            lo = 0;\n        long hi = causal ? i : i + window - 1;\n"
                                "        if (hi > n - 1)\n            hi = n - 1;\n        double m = "
                                "-INFINITY;\n        for (long j = lo; j <= hi; ++j) {\n            "
                                "double dot = 0.0;\n            for (int e = 0; e < d; ++e)\n"
                                "                dot += q[i * d + e] * kk[j * d + e];\n            logit",
                                "(size_t)(2 * window + 1));\n    for (long i = 0; i < n; ++i) {\n"
                                "        long lo = i - window;\n        if (lo < 0)\n"
                                "            lo = 0;\n        long hi = causal ? i : i + window - 1;\n"
                                "        if (hi > n - 1)\n            hi = n - 1;\n        double m = "
                                "-INFINITY;\n        for (long j = lo; j <= hi; ++j) {\n            "
                                "double dot = 0.0;\n            for (int e = 0; e < d; ++e)\n"
                                "                dot += q[i * d + e] * kk[j * d + e];\n            logit"),
    "blocked_lookback_ignored": ("long lo = (i / block - lookback) * block;",
                                 "long lo = (i / block) * block;"),
    "argmax_ties_to_higher": ("            if (x > b1) {\n                b2 = b1;",
                              "            if (x >= b1) {\n                b2 = b1;"),
    "partition_smallest_first": ("    if (x->s > y->s) return -1;\n    if (x->s < y->s) return 1;\n"
                                 "    return (x->t < y->t) ? -1 : (x->t > y->t);\n}\n\n/* Partition",
                                 "    if (x->s < y->s) return -1;\n    if (x->s > y->s) return 1;\n"
                                 "    return (x->t < y->t) ? -1 : (x->t > y->t);\n}\n\n/* Partition"),
    "local_bwd_softmax_sign": ("double dl = P[j - lo] * (dP[j - lo] - D);",
                               "double dl = P[j - lo] * (dP[j - lo] + D);"),
    "local_bwd_dk_from_keys": ("dk[j * d + e] += scale * dl * q[i * d + e];",
                               "dk[j * d + e] += scale * dl * kk[i * d + e];"),
    "local_bwd_dv_unweighted": ("dv[j * d + e] += P[j - lo] * dout[i * d + e];",
                                "dv[j * d + e] += dout[i * d + e];"),
    "softmax_bwd_sign": ("double dl = P[r * w + s] * (dP[r * w + s] - D);",
                         "double dl = P[r * w + s] * (dP[r * w + s] + D);"),
    "centroid_transposed": ("acc += xhat[t * d + i] * mu[c * d + i];",
                            "acc += xhat[t * d + i] * mu[i * k + c];"),
    "margin_wrong_rank": ("margin[c] = (w < n) ? buf[w - 1].s - buf[w].s : INFINITY;",
                          "margin[c] = (w < n) ? buf[0].s - buf[w].s : INFINITY;"),
    "ema_keys_from_queries": ("orc_normalize(kk + u * n * d, n, d, xhat, NULL);\n            "
                              "orc_cluster_sums(xhat, idx + u * k * w, n, d, k, w, sk);",
                              "orc_normalize(q + u * n * d, n, d, xhat, NULL);\n            "
                              "orc_cluster_sums(xhat, idx + u * k * w, n, d, k, w, sk);"),
    "lse_without_max": ("lse[(long)c * w + r] = m + log(z);", "lse[(long)c * w + r] = log(z);"),
    "query_used_as_key": ("dot += qhat[(long)p[r] * d + i] * khat[(long)p[s] * d + i];\n"
                          "                logit[s]",
                          "dot += qhat[(long)p[r] * d + i] * khat[(long)p[r] * d + i];\n"
                          "                logit[s]"),
    "dv_from_wrong_row": ("dv[(long)p[s] * d + i] += pr * g[i];",
                          "dv[(long)p[r] * d + i] += pr * g[i];"),
    # incremental decode (numpy, oracle/__init__.py)
    "decode_ties_to_higher": ("c = int(np.argmax(s))  ", "c = int(len(s) - 1 - np.argmax(s[::-1]))  ",
                              "__init__.py"),
    "decode_keys_unnormalised": ('keys = cache["k"][b, h, c, :j + 1] * cache["inv"][b, h, c, :j + 1, None]',
                                 'keys = cache["k"][b, h, c, :j + 1]', "__init__.py"),
    "decode_fill_wrong_inv": ("cinv[b, h, c, :w] = inv[b, h, p]", "cinv[b, h, c, :w] = inv[b, h, p] * 0 + 1",
                              "__init__.py"),
    # separately routed queries and keys (numpy)
    "split_keys_from_query_rows": ("logits = scale * (qh[b, h, rq] @ kh[b, h, rk].T)",
                                   "logits = scale * (qh[b, h, rq] @ kh[b, h, rq].T)", "__init__.py"),
    "split_scatter_to_key_tokens": ("np.add.at(out[b, h], rq, (e / z) @ v[b, h, rk])",
                                    "np.add.at(out[b, h], rk, (e / z) @ v[b, h, rk])", "__init__.py"),
    "split_values_from_query_rows": ("np.add.at(out[b, h], rq, (e / z) @ v[b, h, rk])",
                                     "np.add.at(out[b, h], rq, (e / z) @ v[b, h, rq])", "__init__.py"),
    # Jensen-Shannon diagnostic (numpy)
    "js_routed_sees_later_keys": ("keys = members[:r + 1] if causal else members",
                                  "keys = members if causal else members", "__init__.py"),
    "js_window_one_too_long": ("near = (pos <= i) & (pos > i - window) if causal",
                               "near = (pos <= i) & (pos >= i - window) if causal", "__init__.py"),
    "js_without_half": ("js[b, h, c, r] = 0.5 * (kl_p + kl_q)", "js[b, h, c, r] = kl_p + kl_q",
                        "__init__.py"),
    "js_local_unscaled": ("ll = np.where(near, scale_l * (k_l[b, h] @ q_l[b, h, i]), -np.inf)",
                          "ll = np.where(near, (k_l[b, h] @ q_l[b, h, i]), -np.inf)", "__init__.py"),
    "local_decode_window_too_long": ("pos = np.arange(max(0, t - window + 1), t + 1)",
                                     "pos = np.arange(max(0, t - window), t + 1)", "__init__.py"),
}


def _run_pins(oracle_dir):
    env = dict(os.environ, RT_ORACLE_DIR=oracle_dir)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests",
                        "test_oracle_pins.py"), "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def _copy(tmp_path, name, edit=None):
    dst = tmp_path / name
    shutil.copytree(SRC, dst, ignore=shutil.ignore_patterns("*.so*", "__pycache__"))
    if edit is not None:
        old, new = edit[0], edit[1]
        path = dst / (edit[2] if len(edit) > 2 else "rt_oracle.c")
        text = path.read_text()
        assert text.count(old) == 1, f"mutation site not found exactly once: {old!r}"
        path.write_text(text.replace(old, new))
    return str(dst)


def test_unmodified_copy_passes(tmp_path):
    rc, out = _run_pins(_copy(tmp_path, "clean"))
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_error_is_caught(tmp_path, name):
    rc, out = _run_pins(_copy(tmp_path, name, MUTANTS[name]))
    assert rc == 1, f"pins did not catch {name}:\n{out}"
