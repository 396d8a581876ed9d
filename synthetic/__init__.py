"""Seeded synthetic inputs for the tests and the bench.

`synth` draws K/V, queries, page tables and ragged lengths from seeded torch
generators (no NVFP4 arithmetic); `workloads` fills device caches with them
through the library's own append calls.  Nothing on the library path imports
this package.
"""
