"""Measurement helpers for bench.py and the summaries under profiles/.

Not part of the product path: libnmspmv never loads anything from here.
  * nmprobe.hip / probe.py -- libnmprobe: a plain streaming-read kernel (the
    achievable read ceiling), a plain copy of known size (calibrates the
    FETCH_SIZE / WRITE_SIZE counters) and an empty kernel (launch cost);
  * profsummary.py -- summaries of rocprofv3 kernel-trace and counter CSVs.
"""
