"""CPU oracle (test infrastructure only): see decode_layer_ref.py."""
