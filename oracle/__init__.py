"""CPU oracle for DCA prefill attention -- test infrastructure only.

Only the tests, the package entry file's smoke check and the benchmark's
CPU-baseline leg import this package; the library's compute path never does.
"""
