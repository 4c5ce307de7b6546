"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a temporary copy of ``oracle/reference.py``,
``oracle/mla_drafter.py``, ``oracle/muon.py`` or ``oracle/projection.py``
(a dropped term, a wrong sign, a wrong index, a swapped operand) and runs the
pin suite against that copy in a subprocess: the suite must fail.  Nothing
here touches the GPU or the HIP library.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "reference.py")

MUTANTS = {
    "eps_dropped": ("return x / np.sqrt(ms + eps) * w", "return x / np.sqrt(ms) * w"),
    "weight_dropped": ("return x / np.sqrt(ms + eps) * w", "return x / np.sqrt(ms + eps)"),
    "rope_sign_flipped": ("return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)",
                          "return np.concatenate([a * c + b * s, b * c - a * s], axis=-1)"),
    "rope_pairs_adjacent": ("a, b = x[..., :h], x[..., h:]", "a, b = x[..., 0::2], x[..., 1::2]"),
    "frequency_index": ("inv_freq = np.float64(theta) ** (-2.0 * i / R)",
                        "inv_freq = np.float64(theta) ** (-1.0 * i / R)"),
    "k_v_swapped": ("k[:, g, :] = X[:, g, q_per_kv, :]\n            v[:, g, :] = X[:, g, q_per_kv + 1, :]",
                    "k[:, g, :] = X[:, g, q_per_kv + 1, :]\n            v[:, g, :] = X[:, g, q_per_kv, :]"),
    "q_head_map_transposed": ("q[:, g * q_per_kv + s, :] = X[:, g, s, :]\n            k[:, g, :]",
                              "q[:, s * n_kv + g, :] = X[:, g, s, :]\n            k[:, g, :]"),
    "sectioned_k_v_swapped": ("k = X[:, n_q:n_q + n_kv, :].copy()\n        v = X[:, n_q + n_kv:, :].copy()",
                              "v = X[:, n_q:n_q + n_kv, :].copy()\n        k = X[:, n_q + n_kv:, :].copy()"),
    "norm_over_whole_row": ("ms = np.mean(x * x, axis=-1, keepdims=True)\n    return",
                            "ms = np.mean(x * x, axis=(-2, -1), keepdims=True)\n    return"),
    "bwd_projection_term_dropped": ("dx = r * (a - xhat * np.mean(a * xhat, axis=-1, keepdims=True))",
                                    "dx = r * a"),
    "bwd_rotation_not_inverted": ("u = g if phi is None else rope_rotate_half_inverse(g, phi)",
                                  "u = g if phi is None else rope_rotate_half(g, phi)"),
    "bwd_weight_dropped": ("a = w * u", "a = u"),
    "wgrad_uses_raw_x": ("return dx, u * xhat", "return dx, u * x"),
    "latent_rope_part_normed": ("kr = rope_rotate_half(kpe, rope_angles(pos, theta, rope_dim))",
                                "kr = rope_rotate_half(rmsnorm(kpe, 1.0, eps), rope_angles(pos, theta, rope_dim))"),
    "paged_offset_off_by_one": ("return page, pos % page_size", "return page, (pos + 1) % page_size"),
    "rounding_truncates": ("r = (u + np.uint64((1 << 44) - 1) + keep_lsb) >> np.uint64(45)",
                           "r = u >> np.uint64(45)"),
}


# mistakes in the MLA drafter layer oracle, caught by its own pin file
DRAFTER_MUTANTS = {
    "absorb_wrong_head": ('return np.einsum("nhd,hdl->nhl", q_nope, w_uk)',
                          'return np.einsum("nhd,hdl->nhl", q_nope, w_uk[::-1])'),
    "q_rope_not_applied": ("q_pe = _store(rope_rotate_half(q[..., qk_nope_head_dim:], "
                           "rope_angles(pos, theta, qk_rope_head_dim)), storage)",
                           "q_pe = _store(q[..., qk_nope_head_dim:], storage)"),
    "q_nope_rope_parts_swapped": ("q_nope = q[..., :qk_nope_head_dim]", "q_nope = q[..., qk_rope_head_dim:]"),
    "q_a_norm_dropped": ("q_a = _store(rmsnorm(q_a, to_f64(w_q_a_ln, dtype), eps), storage)", "q_a = q_a"),
    "kv_from_unnormed_input": ("kv = _store(xn @ to_f64(w_kv_a, dtype), storage)",
                               "kv = _store(X @ to_f64(w_kv_a, dtype), storage)"),
    "storage_skipped": ('    if storage is None:\n        return x\n', '    return x\n'),
}
DRAFTER_SRC = os.path.join(ROOT, "oracle", "mla_drafter.py")

# mistakes in the per-head Newton-Schulz oracle, caught by its own pin file
MUON_MUTANTS = {
    "ns_coefficient_sign": ("X = a * X + (b * A + c * (A @ A)) @ X", "X = a * X + (b * A - c * (A @ A)) @ X"),
    "ns_polynomial_on_the_right": ("X = a * X + (b * A + c * (A @ A)) @ X", "X = a * X + X @ (b * A + c * (A @ A))"),
    "ns_spectral_normalisation": ("X = X / (np.sqrt(np.sum(X * X)) + eps)", "X = X / (np.linalg.norm(X, 2) + eps)"),
    "scale_inverted": ("return max(1.0, rows / cols) ** 0.5", "return max(1.0, cols / rows) ** 0.5"),
    "blocks_without_v": ("blocks = n_q + 2 * n_kv", "blocks = n_q + n_kv"),
}
MUON_SRC = os.path.join(ROOT, "oracle", "muon.py")

# mistakes in the fused projection oracle, caught by its own pin file
PROJ_MUTANTS = {
    "projection_not_transposed": ("return to_f64(x, dtype) @ to_f64(w_qkv, dtype).T",
                                  "return to_f64(x, dtype) @ to_f64(w_qkv, dtype)[:, :to_f64(x, dtype).shape[1]]"),
    "projection_rows_reversed": ("return to_f64(x, dtype) @ to_f64(w_qkv, dtype).T",
                                 "return to_f64(x, dtype) @ to_f64(w_qkv, dtype)[::-1].T"),
    "v_from_k_heads": ("q[t0:t1], k[t0:t1], v[t0:t1] = qn, kn, v_raw", "q[t0:t1], k[t0:t1], v[t0:t1] = qn, kn, k_raw"),
    "q_norm_uses_k_weight": ("qn = rmsnorm(q_raw, wq, eps)", "qn = rmsnorm(q_raw, wk, eps)"),
    "split_always_sectioned": ("q_raw, k_raw, v_raw = split(Y, kind, n_kv, q_per_kv, D)",
                               "q_raw, k_raw, v_raw = split(Y, \"sectioned\", n_kv, q_per_kv, D)"),
}
PROJ_SRC = os.path.join(ROOT, "oracle", "projection.py")


def _run(name, old, new, tmp, src_path=SRC, pins="test_oracle_pins.py"):
    src = open(src_path).read()
    assert src.count(old) == 1, f"{name}: anchor not found exactly once"
    d = os.path.join(tmp, name)
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    with open(os.path.join(d, "oracle", os.path.basename(src_path)), "w") as f:
        f.write(src.replace(old, new))
    env = dict(os.environ, PYTHONPATH=d + os.pathsep + ROOT, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       cwd=d, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, (r.stdout.strip().splitlines() or [""])[-1]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    jobs = [(n, o, w, SRC, "test_oracle_pins.py") for n, (o, w) in MUTANTS.items()]
    jobs += [(n, o, w, DRAFTER_SRC, "test_oracle_mla_drafter.py") for n, (o, w) in DRAFTER_MUTANTS.items()]
    jobs += [(n, o, w, MUON_SRC, "test_oracle_muon.py") for n, (o, w) in MUON_MUTANTS.items()]
    jobs += [(n, o, w, PROJ_SRC, "test_oracle_projection.py") for n, (o, w) in PROJ_MUTANTS.items()]
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda j: _run(j[0], j[1], j[2], str(tmp_path), j[3], j[4]), jobs))
    survivors = [(n, tail) for n, rc, tail in results if rc != 1]
    assert not survivors, f"mistakes no pin caught (or the run broke): {survivors}"


def test_unmutated_copy_passes(tmp_path):
    # the harness itself: the same run on an unchanged copy must pass
    name, rc, tail = _run("unchanged", "def head_blocks(", "def head_blocks(", str(tmp_path))
    assert rc == 0, tail
    name, rc, tail = _run("unchanged_drafter", "def absorb(", "def absorb(", str(tmp_path), DRAFTER_SRC,
                          "test_oracle_mla_drafter.py")
    assert rc == 0, tail


if __name__ == "__main__":
    sys.exit(pytest.main([__file__, "-q"]))
