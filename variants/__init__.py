"""Comparison variants built beside the library (not part of libspecfold).

``correction``: the pages' attention-state correction for folded rows, used by the tests and
the benchmark to compare it with the library's prefix-partial merge.
"""
