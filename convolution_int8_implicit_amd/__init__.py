"""MI355X-native fused int8 ResNet convolution (placeholder; binding added below)."""
