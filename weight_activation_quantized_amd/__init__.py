"""MI355X-native W4.4A8 output-channel mixed-precision linear layer (MixLLM hot path).

The compute path lives in the HIP/C++ library ``libmixllm.so`` (sources under
``csrc/``, C ABI in ``include/mixllm.h``); ``mixllm`` is its thin Python binding.
``workloads`` draws the seeded synthetic inputs.  Importing the package itself does not
load the library, so host-only tools work without a GPU.
"""
