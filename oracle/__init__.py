"""TEST INFRASTRUCTURE ONLY: the plain CPU oracle of the routed MoE-LoRA layer.

Importable only from the tests, the smoke check and the benchmark's
CPU-baseline leg.  It never imports the HIP library.
"""
