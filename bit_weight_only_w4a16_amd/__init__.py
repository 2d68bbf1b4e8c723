"""MI355X-native W4A16 group-quantized GEMV library (binding loads lazily)."""
