"""Routed-expert (sparse MoE) layer for AMD MI355X (gfx950)."""
