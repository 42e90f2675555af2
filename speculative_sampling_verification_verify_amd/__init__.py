"""MI355X (gfx950) batched speculative-sampling verify step.

The compute path is the HIP library ``libspecverify.so`` (built from
``csrc/``); ``binding`` marshals torch tensors into its C ABI.  ``synth``
makes seeded synthetic inputs.  Importing this package does not load the
library; the first call into ``binding`` does, and fails loudly when it is
missing."""
