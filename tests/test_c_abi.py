"""The library driven from C alone: tests/c_abi/table_9_5.c creates a handle
on its own HIP stream, runs the two steps of the page's worked example
("llm_internals" 9.2.2, Table 9-5) with bs_step, swaps the KV rows with
bs_reorder_kv and reads the best hypothesis with bs_finalize, all through the
C ABI with hipMalloc'd buffers, and checks the page's values."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "table_9_5")


@pytest.mark.gpu
def test_c_program_reproduces_table_9_5():
    if not os.path.exists(EXE):
        import importlib.util
        spec = importlib.util.spec_from_file_location("c_abi_build",
                                                      os.path.join(HERE, "c_abi", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
