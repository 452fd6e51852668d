"""MI355X (gfx950) KV-cache vector codec: Python binding over the C-ABI library libkvq.so."""
