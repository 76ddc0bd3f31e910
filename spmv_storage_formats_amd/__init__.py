"""MI355X sparse matrix-vector multiply-accumulate engine (placeholder; binding follows)."""
