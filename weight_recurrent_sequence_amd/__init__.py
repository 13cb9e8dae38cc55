"""Falcon fast-weight recurrence on MI355X (gfx950): C-ABI library + binding."""
