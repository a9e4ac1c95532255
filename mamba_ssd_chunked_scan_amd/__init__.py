"""libssd: the Mamba-2 SSD chunked scan on AMD Instinct MI355X (gfx950)."""
