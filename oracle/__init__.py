"""ORACLE -- test infrastructure only.

A plain, slow CPU implementation of the TokenButler decode-time path (C99 in
tb_oracle.c, fp64 accumulation, explicit storage roundings) with a ctypes
wrapper. Only tests/, the smoke check and the benchmark's cpu_baseline leg may
import it; the GPU library neither links nor imports anything here.
"""
from .oracle import *  # noqa: F401,F403
from .oracle import build, lib  # noqa: F401
