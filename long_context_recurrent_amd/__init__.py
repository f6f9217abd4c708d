"""MI355X-native diagonal-batching forward for layer-level recurrent memory
transformers (ARMT).  The compute lives in libarmt.so (HIP, gfx950); this
package holds its ctypes binding (``armt``) and a small torch-facing wrapper
(``model.ArmtModel``) that owns device buffers."""

from . import armt  # noqa: F401
