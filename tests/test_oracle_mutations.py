"""The pins must catch plausible mistakes in the oracle.  Each case plants one
mistake in a copy of oracle/fmha_oracle.c (or of oracle/mx.py), builds or
loads it, and runs the matching pins (tests/test_oracle.py, resp.
tests/test_mx_oracle.py) against it in a subprocess: at least one pin must
fail.  CPU only."""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fmha_oracle.c")

MUTATIONS = [
    ("scale dropped", "s_buf[j] = J->scale * dot;", "s_buf[j] = dot;"),
    ("causal bound off by one", "if (J->causal && j > pos) return 0;", "if (J->causal && j >= pos) return 0;"),
    ("window keeps W + 1 keys", "if (J->window > 0 && j <= pos - J->window) return 0;",
     "if (J->window > 0 && j < pos - J->window) return 0;"),
    ("GQA group by modulo", "const int kv = h / (J->n_h / J->n_kv_h);", "const int kv = h % J->n_kv_h;"),
    ("queries at the first positions", "int pos = J->s_k - J->T + i;", "int pos = i;"),
    ("lse without the max", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("no normalisation", "for (int d = 0; d < hd; ++d) orow[d] /= l;", "for (int d = 0; d < hd; ++d) orow[d] *= 1.0;"),
    ("normalised twice", "for (int d = 0; d < hd; ++d) orow[d] /= l;",
     "for (int d = 0; d < hd; ++d) orow[d] /= l * l;"),
    ("V read for the query head", "const uint16_t *vp = J->v + b * J->vs[0] + (int64_t)j * J->vs[1] + kv * J->vs[2];",
     "const uint16_t *vp = J->v + b * J->vs[0] + (int64_t)j * J->vs[1] + h * J->vs[2];"),
    ("K and Q swapped in the head index", "const uint16_t *kp = J->k + b * J->ks[0] + (int64_t)j * J->ks[1] + kv * J->ks[2];",
     "const uint16_t *kp = J->k + b * J->ks[0] + (int64_t)j * J->ks[1] + (J->n_kv_h - 1 - kv) * J->ks[2];"),
    ("partition drops its last key", "int hi = lo + J->split_len < J->s_k ? lo + J->split_len : J->s_k;",
     "int hi = lo + J->split_len - 1 < J->s_k ? lo + J->split_len - 1 : J->s_k;"),
    ("merge weights without the max", "double wgt = exp(lp[p] - mx);", "double wgt = exp(lp[p]);"),
    ("merge keeps empty partitions", "if (lp[p] == -INFINITY) continue;", "if (0) continue;"),
    ("softmax of unshifted scores", "double p = exp(s_buf[j] - m);", "double p = exp(s_buf[j]);"),
]


def _pins_fail_with(name, old, new, workdir):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation '{name}' does not match the oracle source exactly once"
    path = os.path.join(workdir, f"mut_{abs(hash(name))}.c")
    lib = path[:-2] + ".so"
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off", path,
                    "-o", lib, "-lm", "-lpthread"], check=True, capture_output=True)
    env = dict(os.environ, FMHA_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as d:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            rcs = list(ex.map(lambda m: _pins_fail_with(*m, d), MUTATIONS))
    survivors = [m[0] for m, rc in zip(MUTATIONS, rcs) if rc == 0]
    assert not survivors, f"mistakes no pin catches: {survivors}"
    assert all(rc == 1 for rc in rcs), rcs  # 1 = tests failed (not a crash or a usage error)


MX_SRC = os.path.join(ROOT, "oracle", "mx.py")

MX_MUTATIONS = [
    ("round half away from zero", "m = torch.round(torch.ldexp(a, (mbits - e).to(torch.float64)))",
     "m = torch.floor(torch.ldexp(a, (mbits - e).to(torch.float64)) + 0.5)"),
    ("truncate instead of round", "m = torch.round(torch.ldexp(a, (mbits - e).to(torch.float64)))",
     "m = torch.floor(torch.ldexp(a, (mbits - e).to(torch.float64)))"),
    ("no carry into the next binade", "carry = m >= 2 ** (mbits + 1)", "carry = m > 2 ** (mbits + 1)"),
    ("no saturation", "code = torch.where(over, torch.full_like(code, max_code), code)", "code = code"),
    ("shared exponent without emax", "_floor_log2(torch.where(amax > 0, amax, torch.ones_like(amax))) - emax",
     "_floor_log2(torch.where(amax > 0, amax, torch.ones_like(amax)))"),
    ("shared exponent rounded up", "_floor_log2(torch.where(amax > 0, amax, torch.ones_like(amax))) - emax",
     "_floor_log2(torch.where(amax > 0, amax, torch.ones_like(amax))) + 1 - emax"),
    ("nibbles swapped", "codes = (codes[..., 0::2].to(torch.int64) | (codes[..., 1::2].to(torch.int64) << 4))",
     "codes = (codes[..., 1::2].to(torch.int64) | (codes[..., 0::2].to(torch.int64) << 4))"),
    ("subnormals flushed", "e = torch.clamp(e, min=emin)", "e = torch.clamp(e, min=emin + 1)"),
    ("exponent bias off by one", "bias = 1 - emin", "bias = 2 - emin"),
]


def _mx_pins_fail_with(name, old, new, workdir):
    src = open(MX_SRC).read()
    assert src.count(old) >= 1, f"mutation '{name}' does not match oracle/mx.py"
    path = os.path.join(workdir, f"mx_mut_{abs(hash(name))}.py")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    env = dict(os.environ, FMHA_ORACLE_MX=path)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_mx_oracle.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_every_planted_mx_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as d:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            rcs = list(ex.map(lambda m: _mx_pins_fail_with(*m, d), MX_MUTATIONS))
    survivors = [m[0] for m, rc in zip(MX_MUTATIONS, rcs) if rc == 0]
    assert not survivors, f"mistakes no pin catches: {survivors}"
    assert all(rc == 1 for rc in rcs), rcs
