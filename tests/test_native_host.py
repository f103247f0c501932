"""Native host-side safety nets (CPU; no GPU needed).

- Address replay: the attention kernel's own tile-addressing functions
  (csrc/attn_geometry.h) evaluated on the host for every workload's sequence
  length and ragged tail, contiguous and (B, N, H, D)-strided layouts, and the
  2^24-element token-stride limit: every global read inside a valid row of the
  head, every LDS write and read inside its tile, the LDS fill a bijection
  (tests/native/addr_replay.cpp). Two planted variants must fail it. The
  same program checks the launch's workgroup -> (head, query block) mapping:
  every item taken exactly once, rounds of consecutive items per XCD, XCD
  loads within one chunk of each other; a planted mapping bug must fail it.
- Sanitizer build: libsparge's host code (api.cpp, noalloc.hip) built with
  AddressSanitizer and UndefinedBehaviorSanitizer and driven through every
  rejection path and host helper (tests/native/abi_host_check.cpp).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "block_sparse_attention_sparge_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is needed to build the host checks")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.fixture(scope="module")
def replay(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("native") / "addr_replay")
    rc, out = _run([HIPCC, "-std=c++17", "-O1", "-o", exe, os.path.join(NATIVE, "addr_replay.cpp")])
    assert rc == 0, out
    return exe


# (D, N, token stride): the five workloads contiguous and (B, N, H, D)-strided,
# the edge lengths around one key block, and the largest token stride accepted.
WORKLOADS = [(64, 1024, 64), (128, 32760, 128), (64, 17776, 64), (128, 75600, 128), (128, 119056, 128),
             (128, 32760, 12 * 128), (64, 17776, 30 * 64), (128, 75600, 40 * 128), (128, 119056, 24 * 128)]
EDGES = [(d, n, d) for d in (64, 128) for n in (1, 2, 63, 64, 65, 127, 128, 129, 191, 700)]
STRIDE_LIMIT = [(128, 65, 1 << 24), (64, 130, 1 << 24), (128, 129, (1 << 24) - 8)]


def test_address_replay(replay):
    args = [str(x) for case in WORKLOADS + EDGES + STRIDE_LIMIT for x in case]
    rc, out = _run([replay] + args)
    assert rc == 0, out
    assert f"{len(WORKLOADS + EDGES + STRIDE_LIMIT)} cases, 0 failures" in out


@pytest.mark.parametrize("plant", ["tail", "swizzle"])
def test_address_replay_catches_planted_mistakes(replay, plant):
    rc, out = _run([replay, "--plant", plant, "64", "17776", "64", "128", "1000", "128"])
    assert rc != 0 and "FAIL" in out


# (items, round): every workload's B * H * ceil(N / 128) with the chunk the
# kernel uses for its head dimension (64 at D=128, 32 at D=64), other chunk
# sizes, and small and boundary counts.
MAP_CASES = [(2 * 8, 32), (12 * 256, 64), (60 * 139, 32), (40 * 591, 64), (24 * 931, 64),
             (1, 64), (1, 32), (255, 32), (256, 32), (257, 32), (511, 64), (512, 64), (513, 64),
             (60 * 139, 128), (40 * 591, 128)]


def test_workgroup_mapping(replay):
    args = [str(x) for case in MAP_CASES for x in case]
    rc, out = _run([replay, "--map"] + args)
    assert rc == 0, out
    assert f"{len(MAP_CASES)} cases, 0 failures" in out


def test_workgroup_mapping_catches_planted_mistake(replay):
    rc, out = _run([replay, "--map", "--plant", "deal", "3072", "64", "23640", "64"])
    assert rc != 0 and "FAIL" in out


def test_sanitized_host_abi(tmp_path):
    """ASan + UBSan on the library's host code; device code built as usual."""
    from block_sparse_attention_sparge_amd.build import SOURCES
    build = os.path.join(ROOT, "_build")
    sanitized = ("api.cpp", "noalloc.hip")          # the library's host code, built below
    objs = [os.path.join(build, os.path.splitext(s)[0] + ".o") for s in SOURCES if s not in sanitized]
    if not all(os.path.exists(o) for o in objs):
        from block_sparse_attention_sparge_amd.build import build as build_lib
        build_lib(verbose=False)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    common = ["-std=c++17", "-O1", "-g", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include")]
    out_objs = []
    for src in sanitized:
        obj = str(tmp_path / (src + ".o"))
        rc, out = _run([HIPCC] + common + ["-fPIC", "-x", "hip", "--offload-arch=gfx950"] + san +
                       ["-c", os.path.join(CSRC, src), "-o", obj])
        assert rc == 0, out
        out_objs.append(obj)
    drv = str(tmp_path / "abi_host_check.o")
    rc, out = _run([HIPCC, "-std=c++17", "-O1", "-g"] + san + ["-c", os.path.join(NATIVE, "abi_host_check.cpp"),
                                                               "-o", drv])
    assert rc == 0, out
    exe = str(tmp_path / "abi_host_check")
    rc, out = _run([HIPCC, "--offload-arch=gfx950"] + san + ["-o", exe, drv] + out_objs + objs)
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and "0 unexpected results" in out, out
