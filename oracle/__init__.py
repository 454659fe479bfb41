"""CPU oracle for the ReplaySSM decode path -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and the two share no
code: the only thing both sides consume is the seeded inputs from ``synth``.

Contents
  core     float64 eager recurrences (Mamba-2's and the gated delta rule's)
           and the storage quantisers (plain C,
           ``replay_oracle.c``, loaded with ctypes; built with gcc on first use)
  forms    the history / checkpoint / output-only rewritings and the segment
           decay, written from their definitions (self-check forms)
  ring     the integer ring-buffer model (pointer, base, error bits)
  runs     the call schedules (standard decode, speculative verify) and the
           dual-precision emulation, driven by the eager recurrence

Parity status of every function is listed in its module docstring.
"""
from .core import (build, lib, threads, set_threads, widen, eager, eager_gdn, bf16_encode, bf16_decode,
                   e4m3_encode, e4m3_decode, quant_heads_e4m3)
from . import forms, ring, runs

__all__ = ["build", "lib", "threads", "set_threads", "widen", "eager", "eager_gdn", "bf16_encode", "bf16_decode",
           "e4m3_encode", "e4m3_decode", "quant_heads_e4m3", "forms", "ring", "runs"]
