"""libtreeverify: target-side speculative tree verification on MI355X.

The compute lives in the HIP library ``libtreeverify.so`` (sources under
``csrc/``); ``binding`` wraps its C ABI for torch tensors and ``workloads``
draws seeded synthetic inputs.  Importing this package loads nothing; the
library is opened on the first call into ``binding``.
"""

__version__ = "0.1.0"
