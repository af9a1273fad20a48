"""The boundary is plain C, and the oracle stays apart from the product."""

import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_plain_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text(textwrap.dedent(f"""
        #include "{ROOT}/include/qlora.h"
        int main(void) {{
          qlora_nf4_desc d = {{4096, 4096, 64, 256, QLORA_TABLE_NF4}};
          size_t a, b, c;
          (void)qlora_nf4_sizes(&d, &a, &b, &c);
          qlora_adamw_hparams h = {{1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 1.0f, 1}};
          (void)h;
          return QLORA_OK + QLORA_W_BF16 * 0 + QLORA_TABLE_UNIFORM * 0;
        }}
    """))
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-fsyntax-only", str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_oracle_imports_nothing_of_the_product():
    code = ("import sys; sys.path.insert(0, %r); import oracle, oracle.nf4, oracle.lora, oracle.optim, oracle.bf16; "
            "bad = [m for m in sys.modules if m.startswith('nf4_bit_quantized_amd')]; "
            "assert not bad, bad; print('ok')" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
