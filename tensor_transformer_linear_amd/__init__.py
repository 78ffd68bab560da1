"""MI355X-native tensor-parallel sharded linear layers (one rank's share, simulated ranks in one HBM).

The compute path is the HIP library ``libttl.so`` built from ``csrc/`` and reached through
``tensor_transformer_linear_amd.ttl`` (ctypes marshalling only).  Importing this package does not
load the library; importing ``ttl`` does, and raises if it has not been built.
"""

__all__ = ["ttl", "workloads"]
