"""The oracle's pins catch plausible mistakes: each case below plants one
mistake in a scratch copy of ``oracle/`` (never in the repository's copy),
runs the pin tests against that copy in a child process and requires at
least one of them to fail.  A mistake that every pin accepts would mean the
oracle is pinned only by itself there.

The planted mistakes: the GQA head map, the causal rule and the query
position ([engine] "03 Correctness, and the bugs a real model found"), the
score scale, K read for V and the in-block offset ([pytorch] "Compute
reference attention without hiding the layout"), the int8 constant, rounding
and dequantisation ([engine] "INT8 KV cache design"), LIFO order and the
copy-on-write threshold ([nanoserve] "What I learned"; [pytorch] "Map the
PyTorch design to vLLM PagedAttention"), the window edge ([pytorch]
"PagedAttention vs sliding-window attention, RadixAttention, and SSMs"),
and the prefix cache and scheduler rules ([manager] "Step 4: The Prefix Tree
(Radix Trie)", "Step 2: The Block Pool"; [engine] "02 The engine").
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the pins: every oracle-only test (none of them calls the HIP path)
PINS = [
    "tests/test_oracle_pins.py",
    "tests/test_sched.py::test_oracle_follows_the_hand_trace",
    "tests/test_prefix_sched_trace.py::test_oracle_prefix_scheduler_follows_the_hand_trace",
    "tests/test_prefix.py::test_lru_subtree_eviction_trace",
]

# (name, file under oracle/, text, replacement)
MUTATIONS = [
    ("gqa map q_head % Hkv", "attention.py", "Ke = np.repeat(Kc, G, axis=1)", "Ke = np.tile(Kc, (1, G, 1))"),
    ("causal mask off by one", "attention.py", "hidden = keys > P", "hidden = keys >= P"),
    ("score scale dropped", "attention.py", "Ke) * float(scale)", "Ke)"),
    ("query position off by one", "attention.py", "int(kv_len) - int(q_len) + np.arange", "int(kv_len) - int(q_len) - 1 + np.arange"),
    ("K read for V", "attention.py", "Vc = gather(pool_v,", "Vc = gather(pool_k,"),
    ("shifted in-block offset", "attention.py", "offs = pos % block_size", "offs = (pos + 1) % block_size"),
    ("dequant scale dropped in the gather", "attention.py", "if scales is not None:", "if False:"),
    ("window edge off by one", "attention.py", "keys < P - int(window) + 1", "keys < P - int(window)"),
    ("int8 constant 128", "kv_write.py", "s = np.float16(amax / f32(127.0))", "s = np.float16(amax / f32(128.0))"),
    ("int8 truncation", "kv_write.py", "np.clip(np.rint(x / f32(s))", "np.clip(np.trunc(x / f32(s))"),
    ("int8 replay drops the old scale", "kv_write.py", "x[:o] = codes_bd[:o].astype(f32) * f32(scale)", "x[:o] = codes_bd[:o].astype(f32)"),
    ("FIFO instead of LIFO", "paging.py", "b = self.stack.pop()\n        self.refs[b] = 1", "b = self.stack.pop(0)\n        self.refs[b] = 1"),
    ("copy-on-write threshold", "paging.py", "elif self.pool.refs[table[lb]] > 1:", "elif self.pool.refs[table[lb]] > 2:"),
    ("admission ignores cached blocks", "scheduler.py", "self.st.pool.num_free + self.st.pool.num_cached - self._owed()", "self.st.pool.num_free - self._owed()"),
    ("admission ignores owed blocks", "scheduler.py", "owed += lifetime_blocks(r, self.bs) - held", "owed += 0"),
    ("first step recomputes the cached prefix", "scheduler.py", "r.first_rows = r.prompt - len(cached) * self.bs", "r.first_rows = r.prompt"),
    ("prompts never published", "scheduler.py", "            if r.tokens:\n                self.st.pool.publish", "            if False:\n                self.st.pool.publish"),
    ("match may cover the whole prompt", "prefix.py", "range((len(tokens) - 1) // block_size)", "range(len(tokens) // block_size)"),
    ("eviction most recently released first", "prefix.py", "self._evict(next(iter(self.cached)))", "self._evict(next(reversed(self.cached)))"),
    ("eviction leaves the subtree", "prefix.py", "order += list(order[i].children.values())", "pass"),
    ("released published blocks freed at once", "prefix.py", "            if b in self.node_of:\n                self.cached[b] = True", "            if False:\n                self.cached[b] = True"),
]


def _scratch_tree(dst):
    for d in ("oracle", "synthetic", "tests"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d),
                        ignore=shutil.ignore_patterns("__pycache__", "*.pyc"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), dst)
    # the native scheduler is imported by two of the pin files (their native tests are not run)
    os.symlink(os.path.join(ROOT, "paged_kv_cache_47_amd"), os.path.join(dst, "paged_kv_cache_47_amd"))


def _run_pins(tree):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *PINS], cwd=tree, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-400:]


def test_the_pins_pass_on_the_unmodified_copy(tmp_path):
    tree = str(tmp_path / "clean")
    _scratch_tree(tree)
    rc, tail = _run_pins(tree)
    assert rc == 0, tail


def test_every_planted_mistake_fails_a_pin(tmp_path):
    trees = []
    for i, (name, fname, old, new) in enumerate(MUTATIONS):
        tree = str(tmp_path / f"m{i}")
        _scratch_tree(tree)
        path = os.path.join(tree, "oracle", fname)
        with open(path) as f:
            src = f.read()
        assert src.count(old) == 1, f"{name}: the text to mutate is not unique in oracle/{fname}"
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        trees.append((name, tree))
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda nt: (nt[0], _run_pins(nt[1])), trees))
    survived = [name for name, (rc, _) in results if rc == 0]
    assert not survived, f"mistakes no pin catches: {survived}"
    # a failure must come from a failing assertion, not from a broken copy
    broken = [name for name, (rc, tail) in results if rc not in (1,)]
    assert not broken, f"pin runs that did not fail cleanly: {broken}"
