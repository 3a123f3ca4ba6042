"""Measurement helpers beside bench.py (not part of the library).

``profiling``: maps the library's kernel roles to rocprofv3 names, turns
rocprofv3 CSV output into the summaries under profiles/, and fingerprints
the sources a kernel is built from.  ``hbm_copy_probe``: a plain device copy
of known size that calibrates the HBM traffic counters.
"""
