"""Plant plausible mistakes in copies of the CPU oracle and check that the pins catch
every one (CPU only).  The real oracle is never modified: each mutant is a patched
copy built into a temporary directory."""
import ctypes
import functools
import importlib.util
import os
import subprocess
import types

import numpy as np
import pytest

import oracle
from oracle import oracle as oracle_py
from oracle_pins import ALL_PINS

ORACLE_DIR = os.path.dirname(oracle.__file__)
C_SRC = os.path.join(ORACLE_DIR, "gmla_oracle.c")
PY_SRC = os.path.join(ORACLE_DIR, "oracle.py")

# (name, exact text in the source, replacement)
C_MUTANTS = [
    ("scale dropped", "s[j] = c->scale * dot;", "s[j] = dot;"),
    ("scale squared", "s[j] = c->scale * dot;", "s[j] = c->scale * c->scale * dot;"),
    ("no position offset", "const int64_t t = i + (c->Tk - c->Tq);", "const int64_t t = i;"),
    ("diagonal masked", "const int64_t last = c->causal ? t : c->Tk - 1;",
     "const int64_t last = c->causal ? t - 1 : c->Tk - 1;"),
    ("causal flag ignored", "const int64_t last = c->causal ? t : c->Tk - 1;",
     "const int64_t last = t;"),
    ("exp sign flipped", "s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    ("not normalised", "for (int64_t j = 0; j <= last; ++j) s[j] /= z;", ""),
    ("keys used as values", "const double* vj = c->v + j * c->ldv;",
     "const double* vj = c->k + j * c->ldk;"),
    ("value column fixed", "o[d] += s[j] * vj[d];", "o[d] += s[j] * vj[0];"),
    ("query row by list position", "const double* qi = c->q + i * c->ldq;",
     "const double* qi = c->q + r * c->ldq;"),
    ("lse without max", "if (c->lse) c->lse[r] = m + log(z);", "if (c->lse) c->lse[r] = log(z);"),
    ("linear transposed W", "acc += xi[kk] * wj[kk];", "acc += xi[kk] * c->w[kk * c->N + j];"),
    ("linear drops last term", "for (int64_t kk = 0; kk < c->K; ++kk) acc += xi[kk] * wj[kk];",
     "for (int64_t kk = 0; kk + 1 < c->K; ++kk) acc += xi[kk] * wj[kk];"),
    ("gate sign flipped", "out[i] = o[i] / (1.0 + exp(-g[i]));", "out[i] = o[i] / (1.0 + exp(g[i]));"),
    ("gate is 1 - sigmoid", "out[i] = o[i] / (1.0 + exp(-g[i]));",
     "out[i] = o[i] - o[i] / (1.0 + exp(-g[i]));"),
]

PY_MUTANTS = [
    ("gate after output projection",
     "    gated = gate(G, Ot, lib)\n    Y = linear(gated, Wo, nthreads, lib)\n",
     "    gated = Ot\n    Y = gate(G, linear(Ot, Wo, nthreads, lib), lib)\n"),
    ("interleaved heads", "sl = slice(h * Dh, (h + 1) * Dh)", "sl = slice(h, dm, num_heads)"),
    ("scale 1/D_h", "Ot[b, :, sl] = attend_head(Q[b, :, sl], K[b, :, sl], V[b, :, sl], 1.0 / np.sqrt(Dh),",
     "Ot[b, :, sl] = attend_head(Q[b, :, sl], K[b, :, sl], V[b, :, sl], 1.0 / Dh,"),
    ("values from W_k", "V = linear(C, Wv, nthreads, lib)", "V = linear(C, Wk, nthreads, lib)"),
    ("keys from W_v", "K = linear(C, Wk, nthreads, lib)", "K = linear(C, Wv, nthreads, lib)"),
    ("queries from W_g", "Q = linear(Xr, Wq, nthreads, lib)", "Q = linear(Xr, Wg, nthreads, lib)"),
    ("cache is K", '"latent_cache": C}', '"latent_cache": K}'),
    ("gate from the context", "G = linear(Xr, Wg, nthreads, lib)", "G = None"),
    ("gate per token", "    gated = gate(G, Ot, lib)\n",
     "    gated = gate(np.repeat(G.mean(axis=-1, keepdims=True), G.shape[-1], -1), Ot, lib)\n"),
]


def _fails(orc):
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(orc)
        except Exception:  # an assertion, or a crash of the broken composition
            failed.append(pin.__name__)
    return failed


def _c_mutant_oracle(tmp_path, find, repl):
    src = open(C_SRC).read()
    assert src.count(find) == 1, f"mutation site not unique: {find!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(find, repl))
    so = str(tmp_path / "libmutant.so")
    oracle.build(src=str(path), out=so)
    lib = oracle.load(so)
    ns = types.SimpleNamespace()
    for name in ("attend_head", "attend", "linear", "gate", "sigmoid", "gated_mla_layer"):
        setattr(ns, name, functools.partial(getattr(oracle_py, name), lib=lib))
    return ns


def _py_mutant_oracle(tmp_path, find, repl):
    src = open(PY_SRC).read()
    assert src.count(find) >= 1, f"mutation site missing: {find!r}"
    path = tmp_path / "oracle_mutant.py"
    path.write_text(src.replace(find, repl).replace("_HERE = os.path.dirname(os.path.abspath(__file__))",
                                                    f"_HERE = {ORACLE_DIR!r}"))
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{abs(hash(find))}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_real_oracle_passes_every_pin():
    assert _fails(oracle) == []


@pytest.mark.parametrize("name,find,repl", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_c_mutant_is_caught(tmp_path, name, find, repl):
    failed = _fails(_c_mutant_oracle(tmp_path, find, repl))
    assert failed, f"no pin catches the mutant '{name}'"


@pytest.mark.parametrize("name,find,repl", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_py_mutant_is_caught(tmp_path, name, find, repl):
    failed = _fails(_py_mutant_oracle(tmp_path, find, repl))
    assert failed, f"no pin catches the mutant '{name}'"
