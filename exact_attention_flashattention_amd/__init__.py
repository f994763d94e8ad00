"""Exact causal GQA attention for MI355X (gfx950): prefill and paged decode."""
