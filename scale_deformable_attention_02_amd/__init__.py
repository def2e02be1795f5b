"""MI355X-native multi-scale deformable attention (MSDA) forward core."""
