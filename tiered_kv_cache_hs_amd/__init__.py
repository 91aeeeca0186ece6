"""HiSparse decode hot path on AMD Instinct MI355X (gfx950).

Submodules:
  hisparse  - Python binding of the C ABI (include/hisparse.h), same names;
  session   - sets up pool, buffers and batch for a workload and captures a
              decode step in a hipGraph (used by the benchmark and tests);
  inputs    - seeded synthetic inputs (traces, records, queries);
  build     - compiles libhisparse.so for gfx950.
"""
