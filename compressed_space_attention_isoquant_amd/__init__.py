"""MI355X-native IsoQuant packed-KV quantisation and compressed-space decode attention."""
