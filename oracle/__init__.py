"""CPU oracle for the NHWC conv2d layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product package never does.
"""
