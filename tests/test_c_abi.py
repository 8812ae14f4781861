"""The library driven from C alone, through the C ABI with hipMalloc'd
buffers and no Python in between:
- tests/c_abi/table_9_5.c creates a handle on its own HIP stream, runs the two
  steps of the page's worked example ("llm_internals" 9.2.2, Table 9-5) with
  bs_step, swaps the KV rows with bs_reorder_kv and reads the best hypothesis
  with bs_finalize, and checks the page's values;
- tests/c_abi/verify_and_resume.c checks the verify example of "Blockwise
  Parallel Decoding" (Figure 1) through bs_verify, bs_verify_noalloc and
  bs_verify_ex, and resumes the Table 9-5 search from a snapshot in a new
  handle (bs_state_save / bs_state_load)."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.gpu
@pytest.mark.parametrize("program", ["table_9_5", "verify_and_resume"])
def test_c_program(program):
    exe = os.path.join(HERE, "c_abi", program)
    if not os.path.exists(exe):
        import importlib.util
        spec = importlib.util.spec_from_file_location("c_abi_build",
                                                      os.path.join(HERE, "c_abi", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
