"""MI355X-native Muon (Newton-Schulz) and AdamW optimizer step."""
