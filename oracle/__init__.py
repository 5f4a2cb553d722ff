"""CPU oracle for the GPT training step. Test infrastructure only: imported by
tests/, the smoke check and bench's cpu_baseline leg, never by the product path."""
