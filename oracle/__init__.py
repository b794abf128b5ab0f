"""Plain fp64 CPU oracle for MLA absorbed-path decode (test infrastructure only)."""
