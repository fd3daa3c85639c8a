"""The C ABI is usable from plain C99 (CPU only): the C consumer program
compiles with -Wall -Wextra -Werror against include/spattn.h and HIP's C
runtime API and links to the in-tree library.  Running it needs a GPU
(tests/test_gpu_c_consumer.py)."""
import subprocess

from tests.c import build_consumer


def test_c_consumer_compiles_and_links(tmp_path):
    r = subprocess.run(build_consumer.command(out=str(tmp_path / "abi_rank_share")), capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert (tmp_path / "abi_rank_share").stat().st_size > 0
