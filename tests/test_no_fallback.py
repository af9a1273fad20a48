"""The product path has no CPU fallback: without the built HIP library every
entry point raises, and nothing under ``oracle`` is imported by the package."""

import subprocess
import sys
import textwrap

import pytest


def test_missing_library_raises(tmp_path):
    code = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {str(__import__('os').path.dirname(__import__('os').path.dirname(__file__)))!r})
        import nf4_bit_quantized_amd as q
        q.LIB_PATH = {str(tmp_path / 'absent.so')!r}
        q._lib = None
        for call in (lambda: q.lib(), lambda: q.qlora_nf4_levels(), lambda: q.qlora_nf4_sizes(64, 64)):
            try:
                call()
            except RuntimeError as e:
                assert "not built" in str(e)
            else:
                raise SystemExit("no error without the library")
        assert not any(m == "oracle" or m.startswith("oracle.") for m in sys.modules), "oracle imported"
        print("ok")
    """)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
