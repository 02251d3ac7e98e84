"""CPU oracle of the INT8ConvRot linear layer (test infrastructure only).

Importable only from the tests, the smoke entry point and the benchmark's
CPU-baseline leg; the product path never uses it.
"""
