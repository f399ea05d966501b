"""Byte sizes of the prefill GEMM's per-group buffer resources, compiled on
the host with g++ from the same header the kernel includes
(llama_decoder_block_amd/csrc/buffer_sizes.hpp).  A resource size is a 32-bit
count: it must cover one 32-row group and never the operand's whole height,
which at 524288 tokens of 4096 bf16 features is 2^32 bytes (0 once wrapped)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "llama_decoder_block_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <cstdlib>
#include "buffer_sizes.hpp"
int main(int argc, char** argv) {
  for (int i = 1; i + 2 < argc; i += 3) {
    const int rows = atoi(argv[i]), first = atoi(argv[i + 1]);
    const long long k = atoll(argv[i + 2]);
    const unsigned row_bytes = static_cast<unsigned>(k * 2);
    std::printf("%u\n", lb::group_bytes(rows, first, row_bytes));
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def group_bytes(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("sizes")
    src, exe = d / "sizes.cpp", d / "sizes"
    src.write_text(PROGRAM)
    subprocess.run(["g++", "-std=c++17", "-O1", f"-I{CSRC}", str(src), "-o", str(exe)], check=True)

    def call(*triples):
        args = [str(v) for t in triples for v in t]
        out = subprocess.run([str(exe), *args], check=True, capture_output=True, text=True).stdout
        return [int(x) for x in out.split()]
    return call


def test_group_bytes_at_half_a_million_tokens(group_bytes):
    """M = 524288 tokens: every 32-row group of the activation operand (K =
    4096 for QKV, o and gate/up; K = 14336 for down) is 32 whole rows."""
    M = 524288
    for K in (4096, 14336):
        firsts = [0, 32, M // 2, M - 64, M - 32]
        got = group_bytes(*[(M, f, K) for f in firsts])
        assert got == [32 * K * 2] * len(firsts)
    # the whole-height size the group must not use would wrap to 0 here
    assert (M * 4096 * 2) % (1 << 32) == 0


def test_group_bytes_at_the_operand_end(group_bytes):
    """Groups that run past the last row cover only the rows that exist, and a
    group past the end has size 0 (its loads return zeros)."""
    assert group_bytes((100, 96, 64), (100, 99, 64), (100, 100, 64), (100, 128, 64)) == [4 * 128, 128, 0, 0]
    assert group_bytes((32, 0, 4096), (31, 0, 4096)) == [32 * 8192, 31 * 8192]


def test_largest_k_keeps_a_group_below_4_gib(group_bytes):
    """The host admits K up to 2^26 - 1 for these kernels: one group of that
    width is just under 2^32 bytes."""
    kmax = (1 << 26) - 1
    (b,) = group_bytes((1 << 20, 0, kmax))
    assert b == 32 * kmax * 2 < (1 << 32)
