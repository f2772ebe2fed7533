"""fp64 CPU oracle of the per-hop KV-cache correction (test infrastructure only)."""
