"""The C ABI from plain C: tests/c_abi_check.c (built by __graft_entry__.build()) allocates with the
HIP runtime, runs a compressed step, the same step split at the exchange, an unpack, a dense step, a
two-worker server reduce and several packs on hand-derived worked examples and checks every output for
equality, plus error paths.  No Python binding or torch is involved."""
import os
import subprocess
import tempfile

import pytest

import __graft_entry__ as entry


def test_c_program_compiles_against_the_header():
    """The public header is valid C11 and the program links against the built library."""
    with tempfile.TemporaryDirectory() as d:
        subprocess.run(entry.c_abi_check_command(os.path.join(d, "c_abi_check")), check=True,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)


@pytest.mark.gpu
def test_c_program_runs_worked_examples():
    assert os.path.exists(entry.C_ABI_CHECK), "tests/c_abi_check is missing: run __graft_entry__.build()"
    r = subprocess.run([entry.C_ABI_CHECK], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=120)
    assert r.returncode == 0 and "c_abi_check ok" in r.stdout, r.stdout
