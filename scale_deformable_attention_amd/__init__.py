"""MI355X-native multi-scale deformable attention core (placeholder until the
HIP library lands)."""
