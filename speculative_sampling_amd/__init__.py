"""MI355X-native verify-and-resample step of speculative sampling.

The compute lives in the HIP library ``libspec_verify.so`` (C ABI declared in
``include/spec_verify.h``); ``speculative_sampling_amd.binding`` marshals
torch device tensors into it.  Importing this package loads nothing; the
library is loaded on first use and its absence is an error.
"""
