"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is a copy of the ``oracle`` package with one source edit (a dropped term,
a wrong sign, index or operand), imported under a private name. This runs on the CPU
only and never touches the real oracle.
"""

import importlib.util
import os
import shutil
import sys

import pytest

from tests import oracle_pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTANTS = [
    ("attention.py", "dist = positions[:, None] - keys[None, :]",
     "dist = keys[None, :] - positions[:, None]"),                       # distance sign
    ("attention.py", "visible &= dist <= window - 1", "visible &= dist <= window"),  # window
    ("attention.py", "visible = dist >= 0", "visible = dist >= -1"),     # causal off by one
    ("attention.py", "logits = softmax_scale * (", "logits = ("),         # dropped scale
    ("attention.py", "s = logits + np.transpose(rel, (1, 0, 2))",
     "s = logits - np.transpose(rel, (1, 0, 2))"),                        # bias sign
    ("attention.py", "s = logits + np.transpose(rel, (1, 0, 2))", "s = logits + 0 * rel.mean()"),
    ("attention.py", "rel = bias_rows[:, idx]", "rel = bias_rows[::-1][:, idx]"),  # head order
    ("attention.py", "idx = np.minimum(np.where(visible, dist, 0), dmax)",
     "idx = np.minimum(np.where(visible, dist, 0), dmax - 1)"),           # clamp column
    ("attention.py", "kv = _gather_kv(k_cache, k_scale, page_table[b], keys, g, page_size)",
     "kv = _gather_kv(k_cache, k_scale, page_table[b], keys, (g + 1) % Hkv, page_size)"),
    ("attention.py", "heads = slice(g * G, (g + 1) * G)",
     "heads = slice(g, Hq, Hkv)"),                                        # GQA map h mod Hkv
    ("attention.py", "slot = keys % page_size", "slot = (keys + 1) % page_size"),
    ("attention.py", "phys = np.asarray(page_table_row)[keys // page_size]",
     "phys = np.asarray(page_table_row)[keys // page_size][::-1]"),
    ("attention.py", "positions = L - n + np.arange(n, dtype=np.int64)",
     "positions = L - 1 - np.arange(n, dtype=np.int64)"),                # row order
    ("attention.py", "out[ok] = (w[ok] @ v_vals) / l[ok][..., None]",
     "out[ok] = (w[ok] @ k_vals) / l[ok][..., None]"),                    # wrong operand
    ("attention.py", "out[ok] = (w[ok] @ v_vals) / l[ok][..., None]",
     "out[ok] = (w[ok] @ v_vals)"),                                       # no normalisation
    ("attention.py", "lse[ok] = m[ok] + np.log(l[ok])", "lse[ok] = np.log(l[ok])"),
    ("attention.py", "lse[ok] = m[ok] + np.log(l[ok])", "lse[ok] = m[ok] + np.log2(l[ok])"),
    ("attention.py", "vals = vals * np.asarray(scale)", "vals = vals / np.asarray(scale)"),
    ("attention.py", "lo = 0 if window == 0 else max(0, L - n + 1 - window)",
     "lo = 0 if window == 0 else max(0, L - n + 2 - window)"),
    ("formats.py", "np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    ("formats.py", "subnormal = m / 8.0 * 2.0 ** -6", "subnormal = m / 8.0 * 2.0 ** -7"),
    ("formats.py", "words = bits.astype(np.uint32) << np.uint32(16)",
     "words = (bits.astype(np.uint32) << np.uint32(16)) | np.uint32(1 << 15)"),
    ("combine.py", "w = np.where(np.isneginf(lse_parts), 0.0, np.exp(lse_parts - M))",
     "w = np.where(np.isneginf(lse_parts), 0.0, np.exp(lse_parts))"),
    ("combine.py", "return out / total[..., None], M + np.log(total)",
     "return out / total[..., None], np.log(total)"),
    # KV append and the E4M3 encoder
    ("append.py", "kr = np.where((frac > 0.5) | ((frac == 0.5) & (np.fmod(kr, 2) == 1)), kr + 1, kr)",
     "kr = np.where(frac >= 0.5, kr + 1, kr)"),                          # ties away from zero
    ("append.py", "quantum = np.exp2(e - 3)", "quantum = np.exp2(e - 2)"),      # 2 fraction bits
    ("append.py", "e = np.maximum(e, -6.0)", "e = np.maximum(e, -7.0)"),         # subnormal binade
    ("append.py", "amax / np.float32(E4M3_MAX)", "amax / np.float32(E4M3_MAX - 1)"),   # scale
    ("append.py", "t = L - n + r", "t = L - n + r + 1"),                          # position
    ("append.py", "slot = t % S", "slot = (t + 1) % S"),                          # slot
    ("append.py", "np.float32(-E4M3_MAX), np.float32(E4M3_MAX))",
     "np.float32(-E4M3_MAX), np.float32(E4M3_MAX) * 0 + np.float32(400))"),  # clamp
    ("append.py", "y = (x / scale[..., None]).astype(np.float32)",
     "y = (x * (np.float32(1) / scale[..., None])).astype(np.float32)"),  # reciprocal
    ("append.py", "y = (x / scale[..., None]).astype(np.float32)",
     "y = x.astype(np.float64) / np.where(amax > 0, amax.astype(np.float64) / E4M3_MAX,"
     " 1.0)[..., None]"),                                                 # float64 scale
    ("append.py", "y = (x / scale[..., None]).astype(np.float32)",
     "y = x.astype(np.float64) / scale[..., None].astype(np.float64)"),   # float64 quotient
    # rows per sequence
    ("varlen.py", "o, s = relative_attention(q[cu[b]:cu[b + 1]][None]",
     "o, s = relative_attention(q[cu[b] + 1:cu[b + 1] + 1][None]"),       # row offset
    ("varlen.py", "out[cu[b]:cu[b + 1]] = o[0]", "out[cu[b]:cu[b + 1]] = o[0][::-1]"),
    ("varlen.py", "np.asarray(seq_lens)[b:b + 1], bias",
     "np.asarray(seq_lens)[b:b + 1] + 1, bias"),                          # position
]


def _load_mutant(tmp_path, index, fname, old, new):
    pkg = "oracle_mutant_%d" % index
    dst = tmp_path / pkg
    shutil.copytree(ORACLE_DIR, dst, ignore=shutil.ignore_patterns("__pycache__"))
    path = dst / fname
    src = path.read_text()
    assert src.count(old) == 1, "mutation site not unique: %r" % old
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(pkg, dst / "__init__.py",
                                                  submodule_search_locations=[str(dst)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[pkg] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("index", range(len(MUTANTS)))
def test_mutant_is_caught(tmp_path, index):
    fname, old, new = MUTANTS[index]
    mutant = _load_mutant(tmp_path, index, fname, old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception as exc:                     # an assertion or a crash both count
            caught.append((pin.__name__, type(exc).__name__))
            break
    assert caught, "no pin caught mutant %d: %s -> %s" % (index, old, new)

