"""NVFP4 CPU oracle package (test infrastructure only; never used by the product path)."""
