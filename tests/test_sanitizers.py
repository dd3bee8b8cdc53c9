"""The host range mapper and the C oracle under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

Each is driven by a small program in tests/sanitize/ over the five workload
layouts, an instance-split layout and seeded random layouts (odd sizes,
lone-param buckets, bus-bandwidth padding, N up to 128).  The oracle driver
also runs three steps (one overflowing), a state export / import, the local
reduce and the bucket check on the small ones.  Each driver is built twice
with the host compiler, plainly and with the sanitizers (no recovery); the
sanitized run must end cleanly and print exactly what the plain build prints.

The oracle's range functions, which the GPU parity harness calls from many
host threads at once, also run from 8 threads under ThreadSanitizer
(tests/sanitize/oracle_threads.c): no race may be reported, and the combined
results must equal the same ranges run on one thread.
"""
import os
import random
import subprocess

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
DT = {"f32": 0, "bf16": 1, "f16": 2}
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _cases() -> str:
    lines = []

    def add(params, N, r, bucket, busbw, inst):
        lines.append(f"{N} {r} {bucket} {busbw} {inst} {len(params)}")
        for p in params:
            lines.append(f"{p[0]} {p[1]} {p[2]} {p[3]} {p[4]}")

    for name in ["tiny", "gpt2-small", "llama3-8b", "dense-7b", "llama3-70b"]:
        w = synth.WORKLOADS[name]
        ps = [(p.numel, DT[p.param_dtype], DT[p.grad_dtype], int(p.requires_new_bucket), int(p.hgroup))
              for p in synth.PARAM_LISTS[w.model]()]
        add(ps, w.dp_size, w.dp_rank, w.bucket_size, w.pad_for_high_busbw, 1)
        if name == "gpt2-small":
            add(ps, 16, 11, w.bucket_size, 0, 2)
    rng = random.Random(7)
    combos = [(1, 1), (1, 0), (2, 2), (2, 0), (0, 0)]
    for _ in range(24):
        n = rng.randint(1, 12)
        ps = []
        for _ in range(n):
            numel = rng.randint(1, 5000) if rng.random() < 0.8 else rng.randint(5000, 200_000)
            pd, gd = rng.choice(combos)
            ps.append((numel, pd, gd, int(rng.random() < 0.15), rng.randint(0, 2)))
        N = rng.choice([1, 2, 3, 4, 8, 64, 96, 128])
        inst = 2 if N % 2 == 0 and rng.random() < 0.3 else 1
        add(ps, N, rng.randrange(N), rng.choice([0, 1000, 5000, 40_000]), int(rng.random() < 0.2), inst)
    lines.append("0 0 0 0 0 0")
    return "\n".join(lines) + "\n"


def _build(tmp, name, cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{name} build failed:\n{r.stderr[-3000:]}"
    return os.path.join(tmp, name)


def _run(exe, stdin):
    r = subprocess.run([exe], input=stdin, capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, f"{os.path.basename(exe)} exited {r.returncode}:\n{r.stderr[-4000:]}"
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def _mapper_cmd(tmp, name, extra):
    src = os.path.join(ROOT, "sharded_mixed_precision_amd", "csrc")
    return ["g++", "-std=c++17", "-O1", "-g", *extra, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
            "-I", src, "-I", "/opt/rocm/include", os.path.join(src, "mapper.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "mapper_driver.cpp"), "-o", os.path.join(tmp, name)]


def _oracle_cmd(tmp, name, extra):
    od = os.path.join(ROOT, "oracle")
    return ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", *extra, "-I", od,
            os.path.join(od, "oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm",
            "-o", os.path.join(tmp, name)]


@pytest.fixture(scope="module")
def cases():
    return _cases()


@pytest.mark.timeout(900)
def test_mapper_under_sanitizers(tmp_path, cases):
    tmp = str(tmp_path)
    plain = _build(tmp, "mapper_plain", _mapper_cmd(tmp, "mapper_plain", []))
    san = _build(tmp, "mapper_san", _mapper_cmd(tmp, "mapper_san", SAN))
    a, b = _run(plain, cases), _run(san, cases)
    assert a == b
    assert a.count("rc 0\n") == 30 and "err -1 -1 -1 -1 -1 -1 -1 -1 -1" in a
    assert "grp_bad -5 -5" in a  # kind and hyper-group out of range


@pytest.mark.timeout(900)
def test_oracle_under_sanitizers(tmp_path, cases):
    tmp = str(tmp_path)
    plain = _build(tmp, "oracle_plain", _oracle_cmd(tmp, "oracle_plain", []))
    san = _build(tmp, "oracle_san", _oracle_cmd(tmp, "oracle_san", SAN))
    a, b = _run(plain, cases), _run(san, cases)
    assert a == b
    assert a.count("rc 0\n") == 30
    # the numeric part ran on the small layouts; the third step's +inf was found and skipped
    n_num = a.count("\nexport ")
    assert n_num >= 20 and a.count("overflow ok") == n_num and "BAD" not in a
    assert a.count(" same 1\n") == n_num  # import of an export leaves the state unchanged


def _threads_cmd(tmp, name, extra):
    od = os.path.join(ROOT, "oracle")
    return ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", *extra, "-I", od,
            os.path.join(od, "oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_threads.c"), "-lm",
            "-pthread", "-o", os.path.join(tmp, name)]


@pytest.mark.timeout(600)
def test_oracle_ranges_from_threads_under_tsan(tmp_path):
    tmp = str(tmp_path)
    plain = _build(tmp, "threads_plain", _threads_cmd(tmp, "threads_plain", []))
    tsan = _build(tmp, "threads_tsan", _threads_cmd(tmp, "threads_tsan", ["-fsanitize=thread"]))
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:exitcode=66")
    r = subprocess.run([tsan], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
    a = subprocess.run([plain], capture_output=True, text=True, timeout=300)
    assert a.returncode == 0 and a.stdout == r.stdout
    lines = r.stdout.splitlines()
    assert len(lines) == 6
    for par, ser in zip(lines[0::2], lines[1::2]):
        assert par.startswith("threads") and ser.startswith("serial")
        assert par.split(None, 1)[1] == ser.split(None, 1)[1]  # bit-identical combined results
