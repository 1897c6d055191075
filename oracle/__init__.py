"""fp64 CPU oracle for the fused gated MLP. Test infrastructure only."""
