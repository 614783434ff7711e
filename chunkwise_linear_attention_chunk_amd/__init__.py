"""MI355X-native chunked-prefill forward of the gated delta rule (Gated DeltaNet / KDA)."""
