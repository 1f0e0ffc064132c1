"""CPU oracle for the QLoRA quantized linear layer (test infrastructure only;
see oracle.py)."""
