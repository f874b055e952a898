"""Mutation tests: plant one plausible mistake in a copy of the oracle's C
source, rebuild it, and require at least one pin to fail.  This shows the pins
are sharp enough to catch dropped terms, wrong signs, wrong indices and
transposed operands anywhere in the oracle (no GPU)."""
import os
import shutil
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

# (id, exact text in the oracle, replacement, pins to run: "seq" or "chunk")
MUTATIONS = [
    ("drop_decay", "for (int i = 0; i < dk * dv; ++i) S[i] *= a;", ";", "seq"),
    ("no_exp_on_g", "const double a = exp(J->g[t * J->H_v + h]);",
     "const double a = J->g[t * J->H_v + h] + 1.0;", "seq"),
    ("delta_sign", "kv[j] = b * ((double)vt[j] - kv[j]);",
     "kv[j] = b * ((double)vt[j] + kv[j]);", "seq"),
    ("drop_beta", "const double b = J->beta[t * J->H_v + h];",
     "const double b = 1.0;", "seq"),
    ("transposed_state_read", "kv[j] += S[i * dv + j] * kh[i];",
     "kv[j] += S[j * dv + i] * kh[i];", "seq"),
    ("readout_with_key", "o[j] += S[i * dv + j] * qh[i];",
     "o[j] += S[i * dv + j] * kh[i];", "seq"),
    ("no_q_scale", "l2_normalise(J->q + (t * J->H_k + hk) * dk, dk, J->eps, J->scale, qh);",
     "l2_normalise(J->q + (t * J->H_k + hk) * dk, dk, J->eps, 1.0, qh);", "seq"),
    ("tiled_gqa", "const int hk = h / r;                                   /* [GQA] */",
     "const int hk = h % J->H_k;", "seq"),
    ("v_indexed_by_key_head", "const double *vt = J->v + (t * J->H_v + h) * dv;",
     "const double *vt = J->v + (t * J->H_v + h / r) * dv;", "seq"),
    ("no_k_norm", "l2_normalise(J->k + (t * J->H_k + hk) * dk, dk, J->eps, 1.0, kh);",
     "for (int i = 0; i < dk; ++i) kh[i] = J->k[(t * J->H_k + hk) * dk + i];", "seq"),
    # chunked form
    ("chunk_mask_without_diagonal", "D[a * C + c] = (c <= a) ? exp(G[a] - G[c]) : 0.0;",
     "D[a * C + c] = (c < a) ? exp(G[a] - G[c]) : 0.0;", "chunk"),
    ("chunk_no_state_decay", "S[i * dv + j] = S[i * dv + j] * exp(gl) + acc;",
     "S[i * dv + j] = S[i * dv + j] + acc;", "chunk"),
    ("chunk_cumdecay_without_exp", "acc += M[a * C + c] * B[c] * exp(G[c]) * K[c * dk + i];",
     "acc += M[a * C + c] * B[c] * K[c * dk + i];", "chunk"),
    ("chunk_gdiff_sign", "acc += K[c * dk + i] * exp(gl - G[c]) * VN[c * dv + j];",
     "acc += K[c * dk + i] * exp(G[c] - gl) * VN[c * dv + j];", "chunk"),
    ("chunk_solve_sign", "for (int m = 0; m < a; ++m) acc += M[a * C + m] * X[m * C + c];",
     "for (int m = 0; m < a; ++m) acc -= M[a * C + m] * X[m * C + c];", "chunk"),
    ("chunk_value_without_beta", "for (int c = 0; c < n; ++c) acc += M[a * C + c] * B[c] * V[c * dv + j];",
     "for (int c = 0; c < n; ++c) acc += M[a * C + c] * V[c * dv + j];", "chunk"),
    ("chunk_inter_without_decay", "for (int i = 0; i < dk; ++i) inter += eg * Q[a * dk + i] * S[i * dv + j];",
     "for (int i = 0; i < dk; ++i) inter += Q[a * dk + i] * S[i * dv + j];", "chunk"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("mid,old,new,kind", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, source, mid, old, new, kind):
    assert source.count(old) == 1, f"mutation site for {mid} not found exactly once"
    src = tmp_path / f"{mid}.c"
    src.write_text(source.replace(old, new))
    lib = str(tmp_path / f"lib_{mid}.so")
    oracle.build(str(src), lib)
    if kind == "seq":
        results = {p.__name__: p(lib) for p in pins.SEQUENTIAL_PINS}
    else:
        results = {"chunked_bruteforce": pins.pin_bruteforce(lib, chunk=16),
                   "chunked_vs_sequential": pins.pin_chunked_vs_sequential(lib)}
    failing = [k for k, v in results.items() if not (v < pins.TOL)]
    assert failing, f"no pin caught mutation {mid}: {results}"
