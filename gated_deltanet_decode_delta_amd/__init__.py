"""Gated DeltaNet decode on MI355X (placeholder, binding follows)."""
