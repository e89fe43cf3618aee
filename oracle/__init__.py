"""CPU oracle for the Sparse-BitLinear path -- test infrastructure only.

Importable only by the tests, the smoke check and the benchmark's CPU-baseline
leg; the library never imports it.
"""
