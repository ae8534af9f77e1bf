"""packed_weight_gemv_amd: placeholder, replaced by the binding."""
