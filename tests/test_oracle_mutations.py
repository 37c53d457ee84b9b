"""The oracle's pins catch plausible mistakes.

Each case copies ``oracle/``, ``workloads/`` and the oracle pin tests into a
temporary directory, plants one mistake in the copied oracle (a wrong index,
a dropped term, a swapped operand, an off-by-one), and runs the pin tests on
the copy in a child process.  The pins must fail.  Nothing here touches the
GPU or the HIP path; the mistakes live only in the temporary copy.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    # (id, file, original text, planted mistake, pin files to run)
    ("gqa-map", "attention.py", "g = h // group", "g = h % num_kv_heads", ["test_oracle_attention.py"]),
    ("causal-off-by-one", "attention.py", "(t <= pos)", "(t < pos)", ["test_oracle_attention.py"]),
    ("drop-cached-offset", "attention.py", "pos = c + np.arange(n)[:, None]", "pos = np.arange(n)[:, None]", ["test_oracle_attention.py"]),
    ("drop-scale", "attention.py", "s = scale * (Q[:, h, :] @ K[:, g, :].T)", "s = (Q[:, h, :] @ K[:, g, :].T)", ["test_oracle_attention.py"]),
    ("values-from-keys", "attention.py", "(w @ V[:, g, :])", "(w @ K[:, g, :])", ["test_oracle_attention.py"]),
    ("normalise-over-all-rows", "attention.py", "/ w.sum(axis=1, keepdims=True)", "/ w.sum()", ["test_oracle_attention.py"]),
    ("row-in-block", "attention.py", "cache[blocks, :, t % block_size, :]", "cache[blocks, :, (t + 1) % block_size, :]", ["test_oracle_cache.py"]),
    ("merge-unscaled-sum", "attention.py", "np.exp(m - M) * l for", "l for", ["test_oracle_attention.py"]),
    ("block-count", "blocks.py", "return -(-n_tokens // block_size)", "return n_tokens // block_size + 1", ["test_oracle_blocks.py"]),
    ("cow-private-block", "alloc.py", "j not in copied and self.refcount[table[j]] > 1:\n                old", "j not in copied and self.refcount[table[j]] >= 1:\n                old", ["test_oracle_alloc.py"]),
    ("cow-keeps-ref", "alloc.py", "self.refcount[old] -= 1", "pass", ["test_oracle_alloc.py"]),
    ("fork-drops-partial-block", "alloc.py", "[: blocks_needed(share_tokens, self.block_size)]", "[: share_tokens // self.block_size]", ["test_oracle_alloc.py"]),
    ("lifo-reuse", "alloc.py", "self.free.append(b)", "self.free.appendleft(b)", ["test_oracle_alloc.py"]),
    ("fnv-prime", "prefix.py", "FNV_PRIME = 0x100000001B3", "FNV_PRIME = 0x100000001B5", ["test_oracle_prefix.py"]),
    ("fnv-mul-before-xor", "prefix.py", "h ^= byte\n        h = (h * FNV_PRIME) & _MASK", "h = (h * FNV_PRIME) & _MASK\n        h ^= byte", ["test_oracle_prefix.py"]),
    ("hash-drops-parent", "prefix.py", "data = int(parent).to_bytes(8, \"little\") + b\"\".join(", "data = b\"\".join(", ["test_oracle_prefix.py"]),
    ("token-low-byte", "prefix.py", "(int(t) & 0xFFFFFFFF).to_bytes(4, \"little\")", "(int(t) & 0xFF).to_bytes(4, \"little\")", ["test_oracle_prefix.py"]),
    ("lookup-caches-all", "alloc.py", "for b in range(max(n - 1, 0) // B):", "for b in range(n // B):", ["test_oracle_prefix.py"]),
    ("lookup-keeps-free", "alloc.py", "                self.free.remove(blk)\n", "                pass\n", ["test_oracle_prefix.py"]),
    ("no-eviction", "alloc.py", "        b = self.free.popleft()\n        self._unregister(b)", "        b = self.free.popleft()", ["test_oracle_prefix.py"]),
    ("register-overwrites", "alloc.py", "if blk not in self.reg and h not in self.cache:", "if blk not in self.reg:", ["test_oracle_prefix.py"]),
    ("in-place-write-kept", "alloc.py", "self._unregister(table[j])   # written in place", "pass   # written in place", ["test_oracle_prefix.py"]),
    ("e4m3-bias", "quant.py", "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)", "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)", ["test_oracle_quant.py"]),
    ("e4m3-subnormal-step", "quant.py", "q_sub = np.rint(a * 2.0 ** 9)", "q_sub = np.rint(a * 2.0 ** 8)", ["test_oracle_quant.py"]),
    ("round-half-up", "quant.py", "q = np.rint((2.0 * m - 1.0) * 8.0)", "q = np.floor((2.0 * m - 1.0) * 8.0 + 0.5)", ["test_oracle_quant.py"]),
    ("no-carry", "quant.py", "    E = E + carry\n", "", ["test_oracle_quant.py"]),
    ("scale-not-minimal", "quant.py", "e = np.where(safe <= np.ldexp(E4M3_MAX, e - 1), e - 1, e)", "e = e + 1", ["test_oracle_quant.py"]),
    ("v-not-transposed", "quant.py", "return rows * D + d if kind == \"k\" else d * block_size + rows", "return rows * D + d", ["test_oracle_quant.py"]),
    ("scale-bias", "quant.py", "e = np.asarray(exp_codes, dtype=np.int64) - SCALE_BIAS", "e = np.asarray(exp_codes, dtype=np.int64) - SCALE_BIAS - 1", ["test_oracle_quant.py"]),
    ("bf16-shift", "numerics.py", "x.astype(np.uint32) << np.uint32(16)", "x.astype(np.uint32) << np.uint32(15)", ["test_oracle_numerics.py", "test_oracle_attention.py"]),
    ("bf16-low-half", "numerics.py", "x.astype(np.uint32) << np.uint32(16)", "x.astype(np.uint32)", ["test_oracle_numerics.py", "test_oracle_attention.py"]),
    ("v-from-k", "cache.py", "v_cache[blocks, :, rows, :] = np.asarray(v)[keep]", "v_cache[blocks, :, rows, :] = np.asarray(k)[keep]", ["test_oracle_cache.py"]),
]


@pytest.mark.parametrize("mid,fname,old,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, mid, fname, old, new, pins):
    for d in ("oracle", "workloads"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ["conftest.py", "helpers.py"] + pins:
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    target = tmp_path / "oracle" / fname
    src = target.read_text()
    assert src.count(old) >= 1, f"mutation site for {mid} not found; update the mutation list"
    target.write_text(src.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         *[f"tests/{p}" for p in pins]],
        cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"planted mistake {mid} passed every pin:\n{res.stdout[-2000:]}"
    assert "failed" in res.stdout or "error" in res.stdout.lower()
