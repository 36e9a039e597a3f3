"""MI355X-native verify-side path of budget-aware tree speculative decoding.

Submodules:
  workload  seeded synthetic inputs (no step of the path)
  binding   ctypes binding over the HIP library libtreedraft.so
"""
__all__ = ["workload", "binding"]
