"""Oracle package: plain, slow, obviously correct CPU references.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import anything from here. The product path
(the HIP library and its Python binding) never imports, links or executes this
package, and shares no code with it.

Contents
--------
attn_ref.c / ref.py
    fp64 softmax-attention forward and backward, the textbook definition written
    out (the pages only name "partial gradients dQ, dK, dV" of tiled attention:
    DASH, zskr.cn explainer section 2.1). Pinned by finite differences, PyTorch
    float64 autograd, closed-form identities and special cases (tests/test_oracle.py).
schedules.py
    The pages' tile orders (serialized ascending, descending Q tiles, cyclic
    shift, symmetric shift) written from their prose, and each dQ tile's
    accumulation order. Pinned by golden n=4 tables, coverage and conflict checks.
dagsim.py
    The pages' DAG model of compute/reduce stages and an exact critical-path
    simulator. Pinned by the pages' closed forms and Lemma 1.
"""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_ref.so")
SRC_PATH = os.path.join(_HERE, "attn_ref.c")


def build(force: bool = True) -> str:
    """Compile attn_ref.c with gcc into oracle/libattn_ref.so (OpenMP, plain fp64).

    -ffp-contract=off keeps every multiply and add a separate IEEE operation, so
    the oracle's arithmetic is exactly what its source says.
    """
    if not force and os.path.exists(LIB_PATH) and os.path.getmtime(LIB_PATH) >= os.path.getmtime(SRC_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-o", tmp, SRC_PATH, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH
