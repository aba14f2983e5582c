"""CPU oracle for the paged KV cache decode path (test infrastructure only)."""
