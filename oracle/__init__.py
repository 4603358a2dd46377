"""CPU float64 oracle (test infrastructure only; see lora_oracle.py)."""
