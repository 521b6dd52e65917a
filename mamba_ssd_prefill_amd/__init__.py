"""MI355X-native Mamba-2 SSD chunked prefill (forward): Python binding over libmamba_ssd.so."""
