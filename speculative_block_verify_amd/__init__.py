"""MI355X-native block-verify forward through NVFP4 mixture-of-experts layers.

The compute path is the HIP shared library built from ``csrc/``; ``api``
binds its C entry points.  ``inputs`` generates seeded synthetic data.
Importing the package loads nothing; ``api`` loads the library on first use.
"""
