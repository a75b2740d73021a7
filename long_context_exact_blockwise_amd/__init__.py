"""MI355X-native forward of one device's share of ring attention.

The HIP library (``libringattn.so``, built from ``csrc/``) holds every step of
the path; ``ringattn`` is the ctypes binding over its C ABI.  Importing this
package does not load the library; the first call into the binding does, and
it raises if the library is missing.
"""
