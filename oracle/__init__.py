"""CPU oracle of the MoE-FFN layer forward -- TEST INFRASTRUCTURE.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package. `moe_ref` is the float64 NumPy/SciPy definition of
the layer; `brute` is an independent pure-Python restatement for tiny inputs
that pins it. Neither shares code with, or imports, the HIP library.
"""
