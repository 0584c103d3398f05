"""gelu_bf16_gemm_amd — an MI355X (gfx950) fused-linear library: Y = act(X W^T + b) with an
in-register epilogue, a LayerNorm+GELU row kernel and an RMSNorm finalize kernel.

The product is ``libfusedops.so`` (C ABI in ``include/fusedops.h``), built from
``csrc/`` by ``python -m gelu_bf16_gemm_amd.build``. ``binding`` is its thin
ctypes binding; ``inputs`` draws the seeded synthetic workloads. Accessing
the binding's entry points through this package loads the library and fails
loudly if it has not been built.
"""

__all__ = ["binding", "inputs", "fusedops_linear_epilogue", "fusedops_layernorm_gelu",
           "fusedops_rmsnorm_finalize", "fusedops_linear_workspace_bytes"]


def __getattr__(name):
    if name in ("fusedops_linear_epilogue", "fusedops_layernorm_gelu", "fusedops_rmsnorm_finalize",
                "fusedops_linear_workspace_bytes", "binding"):
        import importlib
        binding = importlib.import_module(__name__ + ".binding")
        return binding if name == "binding" else getattr(binding, name)
    raise AttributeError(name)
