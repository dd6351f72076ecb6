"""LeapQuant decode for delta-rule linear attention (GDN / KDA) on MI355X."""
