"""The host code of libpa under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tests/asan/bm_driver.cpp is compiled with g++ -fsanitize=address,undefined together
with the block manager (csrc/block_manager.cpp), the C ABI's validation (csrc/api.cpp)
and launcher stubs that abort if reached. The block manager's random operation
sequences of tests/test_block_manager.py then run through the driver, answer for
answer against the reference model in oracle/blocks.py, and the ABI's validation cases
run once; any sanitizer report (out-of-bounds access, use after free, leak, undefined
behaviour) makes the driver exit non-zero and the test fail."""
import os
import shutil
import subprocess

import pytest

import paged_kv_cache_95_amd as pa

from test_block_manager import _random_ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_95_amd", "csrc")
SOURCES = [os.path.join(ROOT, "tests", "asan", "bm_driver.cpp"),
           os.path.join(ROOT, "tests", "asan", "stubs.cpp"),
           os.path.join(CSRC, "block_manager.cpp"), os.path.join(CSRC, "api.cpp")]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("asan") / "bm_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include"] + SOURCES + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in r.stderr.lower() and "cannot find" in r.stderr.lower():
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


class Driver:
    """The block manager behind the sanitizer-built driver process, with the interface
    of paged_kv_cache_95_amd.BlockManager."""

    def __init__(self, exe, num_blocks, block_size, prefix_caching):
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")
        self.p = subprocess.Popen([exe], stdin=subprocess.PIPE, stdout=subprocess.PIPE,
                                  stderr=subprocess.PIPE, text=True, env=env)
        self.block_size = block_size
        assert self.ask(f"create {num_blocks} {block_size} {int(prefix_caching)}") == []

    def ask(self, line):
        self.p.stdin.write(line + "\n")
        self.p.stdin.flush()
        ans = self.p.stdout.readline().split()
        if not ans:
            self.p.wait(timeout=30)
            raise AssertionError(f"driver died on {line!r}: {self.p.stderr.read()[-3000:]}")
        if ans[0] == "err":
            raise pa.PaError(int(ans[1]), line.split()[0])
        assert ans[0] == "ok", ans
        return [int(x) for x in ans[1:]]

    def close(self):
        self.p.stdin.write("quit\n")
        self.p.stdin.flush()
        rc = self.p.wait(timeout=60)
        err = self.p.stderr.read()
        assert rc == 0, f"sanitizer exit {rc}: {err[-3000:]}"
        assert "ERROR: AddressSanitizer" not in err and "runtime error" not in err, err[-3000:]

    @property
    def num_free(self):
        return self.ask("free_count")[0]

    def add_sequence(self, seq_id, token_ids):
        t = [int(x) for x in token_ids]
        return self.ask(f"add {seq_id} {len(t)} " + " ".join(map(str, t)))[0]

    def append(self, seq_id, token_id):
        return tuple(self.ask(f"append {seq_id} {int(token_id)}"))

    def fork(self, parent_id, child_id):
        self.ask(f"fork {parent_id} {child_id}")

    def free(self, seq_id):
        self.ask(f"free {seq_id}")

    def context_len(self, seq_id):
        return self.ask(f"ctx {seq_id}")[0]

    def block_tables(self, seq_ids, max_blocks_per_seq):
        import numpy as np
        ids = [int(x) for x in seq_ids]
        v = self.ask(f"tables {max_blocks_per_seq} {len(ids)} " + " ".join(map(str, ids)))
        n = len(ids) * max_blocks_per_seq
        return (np.array(v[:n], np.int32).reshape(len(ids), max_blocks_per_seq),
                np.array(v[n:], np.int32))

    def slots(self, seq_id, first_pos, count):
        import numpy as np
        return np.array(self.ask(f"slots {seq_id} {first_pos} {count}"), np.int64)

    def refcount(self, block):
        return self.ask(f"ref {block}")[0]


@pytest.mark.parametrize("seed", range(4))
def test_block_manager_ops_under_sanitizers(driver, seed):
    made = []

    def make(n, bs, pc):
        made.append(Driver(driver, n, bs, pc))
        return made[-1]

    _random_ops(seed, nblocks=24, bs=4, steps=200, prefix_caching=seed % 3 != 2, make=make)
    for d in made:
        d.close()


def test_abi_validation_under_sanitizers(driver):
    d = Driver(driver, 4, 16, True)
    assert d.ask("abi") == []
    # error paths of the manager: nothing changes, nothing leaks
    with pytest.raises(pa.PaError):
        d.add_sequence(1, list(range(100)))
    with pytest.raises(pa.PaError):
        d.append(9, 1)
    with pytest.raises(pa.PaError):
        d.slots(1, 0, 5)
    assert d.num_free == 4
    d.close()
